// Internal declarations shared by the f16wm HIP sources (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "f16wm.h"

namespace f16wm {

// Rows of up to F16WM_MAX_MULTI matrices that share k and one activation,
// laid end to end: global row g belongs to matrix m when
// row0[m] <= g < row0[m + 1].
// tile0[m] is the first row tile of matrix m for kernels that give every
// block the rows of one matrix only (filled by the launcher for its tile
// height; tile0[count] is the tile total).
struct RowTable {
    const uint16_t *w[F16WM_MAX_MULTI];
    float *out[F16WM_MAX_MULTI];
    int64_t row0[F16WM_MAX_MULTI + 1];
    int64_t tile0[F16WM_MAX_MULTI + 1];
    int32_t count;
};

// Products of up to F16WM_MAX_MULTI weight matrices that share k and one
// activation block A [n][k]: matrix m has rows[m] rows and output out[m]
// ([n][rows[m]]).  tile0[m] is the first output tile of matrix m (filled by
// the launcher for its tile size), so one launch covers every matrix.
struct GemmTable {
    const uint16_t *w[F16WM_MAX_MULTI];
    float *out[F16WM_MAX_MULTI];
    int64_t rows[F16WM_MAX_MULTI];
    int32_t tile0[F16WM_MAX_MULTI + 1];
    int32_t count;
};

// Independent one-column products, each with its own weight (rows[p] x
// k[p] f16), column a[p] (k[p] values, all f16 or all f32 in one table) and
// output out[p] (rows[p] f32).  tile0[p] is the first row tile of product p
// (filled by the launcher for its tile height; tile0[count] is the total).
// kTableChunk products fit in the 4 KB a kernel's arguments may take.
constexpr int kTableChunk = 96;
struct ProdTable {
    const uint16_t *w[kTableChunk];
    const void *a[kTableChunk];
    float *out[kTableChunk];
    int32_t rows[kTableChunk];
    int32_t k[kTableChunk];
    int32_t tile0[kTableChunk + 1];
    int32_t count;
};
static_assert(sizeof(ProdTable) <= 4096, "kernel arguments stay within 4 KB");

// The output tile `t` of a grouped product with `nct` column tiles: its
// matrix, row tile and column tile.
__device__ __forceinline__ void gemm_tile(const GemmTable &g, int t, int nct, int &m, int &rt, int &ct)
{
    m = 0;
#pragma unroll
    for (int i = 1; i < F16WM_MAX_MULTI; i++)
        if (i < g.count && t >= g.tile0[i]) m = i;
    const int local = t - g.tile0[m];
    rt = local / nct;
    ct = local % nct;
}

// Block b of a grid of `ntiles` blocks runs on XCD b % 8 (round-robin
// dispatch); this hands each XCD a contiguous range of tiles.
__device__ __forceinline__ int xcd_tile(int b, int ntiles)
{
    const int xcd = b & 7, pos = b >> 3, q = ntiles >> 3, rem = ntiles & 7;
    return xcd * q + (xcd < rem ? xcd : rem) + pos;
}

// Compute units of the current device (looked up once per device).
int64_t device_cus();

// Lets kernel `fn` take `bytes` of dynamic LDS on the current device (the
// attribute is set once per device and kernel; later calls only look it up).
void allow_dynamic_lds(const void *fn, int bytes);

// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
hipError_t launch_to_f16(const float *x, uint16_t *y, int64_t count, hipStream_t stream);

// vec_dot order for `ncols` activation columns (column c at a + c*k, output
// of matrix m column c at out[m] + c*rows_m).  The activation is f16 bit
// patterns, or f32 values (f32act) rounded in the kernel exactly as
// launch_to_f16 rounds them.  vec8 needs k % 8 == 0 and 16-byte aligned w[]
// and a.
hipError_t launch_vec_dot(const RowTable &t, int64_t k, const void *a, bool f32act, int64_t ncols,
                          bool vec8, hipStream_t stream);

// vec_dot order for every product of t in one launch.  Every product has
// k % 8 == 0, 16-byte aligned w and a, rows < 2^31, and 16 * 2 * k + 64 KB
// under 2^31 bytes; direct: every k <= kDirectMaxKTable (rows in registers),
// else rows staged in LDS.  f32act: every column is f32, rounded in the
// kernel exactly as launch_to_f16 rounds it.  The launcher fills tile0 and
// fails (hipErrorInvalidConfiguration) past 2^31 - 1 row tiles.
constexpr int64_t kDirectMaxKTable = 576;
constexpr int kTableRowsDirect = 16;   // rows per block, direct kernel
constexpr int kTableRowsLds = 16;      // rows per block, LDS kernel
hipError_t launch_vec_dot_table(ProdTable t, bool direct, bool f32act, hipStream_t stream);

// tinyBLAS order for every matrix of g (rows % 4 == 0, k % 8 == 0, n >= 2
// checked by the caller).  aligned16: every w and a are 16-byte aligned.  The
// activation block a [n][k] is f16 bit patterns, or f32 values (f32act)
// rounded in the kernel exactly as launch_to_f16 rounds them.
hipError_t launch_sgemm(GemmTable g, int64_t k, const void *a, int64_t n, bool aligned16, bool f32act,
                        hipStream_t stream);

// Exact f16 -> f32 of count values, and of rows ids[0..nids) of W (rows x k)
// into out[nids][k] (an id outside [0, rows) gives a row of NaN).
hipError_t launch_widen(const uint16_t *h, float *y, int64_t count, hipStream_t stream);
hipError_t launch_get_rows(const uint16_t *w, int64_t rows, int64_t k, const int64_t *ids, int64_t nids,
                           float *out, hipStream_t stream);

// vec_dot scores of n_head queries against an f16 K cache [n_kv][n_kv_head][d]
// (out [n_head][n_kv]); vec8: d % 8 == 0 and 16-byte aligned kc and q.
hipError_t launch_kq(const uint16_t *kc, int64_t n_kv, int64_t n_kv_head, int64_t d, const uint16_t *q,
                     int64_t n_head, bool vec8, float *out, hipStream_t stream);

// acc[b][i] = f16(fma(v[b][i], w[b], acc[b][i])) and acc[b][i] = f16(acc[b][i] * s[b]);
// vec8: n % 8 == 0 and 16-byte aligned f16 arrays.
hipError_t launch_mad(uint16_t *acc, const uint16_t *v, const float *w, int64_t nvec, int64_t n, bool vec8,
                      hipStream_t stream);
hipError_t launch_scale(uint16_t *acc, const float *s, int64_t nvec, int64_t n, bool vec8, hipStream_t stream);

// fp16 MFMA product of every matrix of g (k % 8 == 0, w and a 16-byte
// aligned).
hipError_t launch_mfma(GemmTable g, int64_t k, const uint16_t *a, int64_t n, hipStream_t stream);

}  // namespace f16wm
