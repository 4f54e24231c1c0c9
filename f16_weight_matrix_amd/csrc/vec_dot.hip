// vec_dot order on gfx950: GEMV (one column), grouped GEMV, and the fallback
// product for shapes that do not take the tinyBLAS path.
//
// The order (bankML page "bankML/f16.rs -- F16 weights, multiplied as the
// shipped ggml b11192 multiplies them", Design notes, "vec_dot"; Matrix
// products for mat_vec_par / mat_vec_multi_par):
//  - chains: element i < 32 * floor(k / 32) goes to chain c = i % 32, and
//    every chain is one sequential f32 FMA chain from +0 in ascending i;
//  - tree: chains c and c + 16 are added, then those sums pairwise by bit 8
//    of c, then by bit 4, then two rounds of neighbour sums (bit 1, then
//    bit 2), leaving one f32;
//  - tail: the k % 32 last products are added to that f32 one by one in
//    binary64 and the double is rounded to f32 once;
//  - out[r] = that value for row r of W against the column, for one or
//    several matrices per launch.
//
// Each of the 32 chains of an element is a sequential FMA chain, so one chain
// lives in one GPU lane for the whole row; the tree is a fixed sequence of
// adds.  With LPR lanes per row, lane q of the row owns the CPL = 32 / LPR
// consecutive chains CPL q .. CPL q + CPL - 1; a tree level pairs chains c
// and c ^ b, across lanes when b >= CPL and inside a lane otherwise
// (vec_dot_order.h).  Every layout holds the same 32 chains and applies the
// same adds, so all give the same bits:
//   vec_dot_direct (k <= 576, k % 8 == 0, 16-byte alignment): 4 lanes per
//         row, each loading the 16 bytes W[r][32t + 8q .. +7] of its chains
//         per step straight into registers.
//   vec_dot_lds (k % 8 == 0, 16-byte alignment): 16 or 32 lanes per row,
//         reading their chains from row stages copied into LDS.
//   vec_dot_v1 (any k, any alignment): 32 lanes per row, lane c loads
//         element 32t + c.
// The products of two f16 values are exact in f32, so each chain step's FMA
// equals an exact product added with one rounding; the widening of f16 inputs
// is exact (v_cvt_f32_f16 / the f16 operands of v_fma_mix_f32, with f16
// subnormals kept).
//
// HBM-bound: 2*k bytes of weight per row, read once, with the activation
// column (2*k bytes) served from cache.
#include "buffer_rsrc.h"
#include "f16_round.h"
#include "kernels.h"
#include "vec_dot_order.h"

namespace f16wm {
namespace {

__device__ __forceinline__ int find_matrix(const RowTable &t, int64_t g)
{
    int m = 0;
#pragma unroll
    for (int i = 1; i < F16WM_MAX_MULTI; i++)
        if (i < t.count && g >= t.row0[i]) m = i;
    return m;
}

// Activation element i as an f16 bit pattern: stored f16, or an f32 value
// rounded here exactly as f16wm_to_f16 rounds it.
template <bool kF32>
__device__ __forceinline__ uint16_t act16(const void *a, int64_t i)
{
    if (kF32) return rne_f16(static_cast<const float *>(a)[i]);
    return static_cast<const uint16_t *>(a)[i];
}

// The k % 32 tail in binary64, ascending, onto the f32 tree result.
template <bool kF32>
__device__ __forceinline__ float add_tail(float v, const uint16_t *w, const void *a, int64_t from,
                                          int64_t k)
{
    double d = (double)v;
    for (int64_t i = from; i < k; i++) {
        const float p = widen(w[i]) * widen(act16<kF32>(a, i));   // exact in f32
        d = d + (double)p;
    }
    return (float)d;
}

// LDS-staged GEMV for k % 8 == 0 and 16-byte aligned rows.
//
// A 256-thread block owns R = 256 / LPR rows.  Each stage copies SC elements
// of every row (16 or 32 KB of weights) plus the matching SC activation elements
// from HBM into LDS with 16-byte loads in which consecutive lanes read
// consecutive bytes of one row (512 B to 4 KB contiguous per row), so every
// wave load is fully coalesced.  The compute lanes then read their chains'
// elements from LDS: lane j of a row owns chains CPL*j .. CPL*j + CPL - 1 and
// per 32-element step reads CPL consecutive halves of the row and of the
// activation.  Two LDS buffers: the next stage's loads are in flight while
// the current stage computes.  Rows are padded to a stride of 64 mod 256
// bytes so the rows read by one LDS instruction fall in different banks.
template <int LPR>
struct LdsCfg {
    static constexpr int R = 256 / LPR;        // rows per block
    static constexpr int CPL = 32 / LPR;       // chains per lane
    // Weight bytes per stage: 16 KB (measured best on MI355X against 8 and
    // 32 KB, with 2 to 8 stages in flight).
    static constexpr int STAGE = 16384;
    static constexpr int SC = STAGE / 2 / R;   // elements per row per stage
    static constexpr int U = SC / 8;           // 16-byte units per row per stage
    static constexpr int UPT = R * U / 256;    // units per thread per stage
    static constexpr int ROWB = SC * 2 + 64;   // LDS row stride, bytes
    static constexpr int WBYTES = R * ROWB;    // weight bytes per LDS buffer
    static constexpr int BUFB = WBYTES + SC * 2;
    static_assert(U <= 256, "one 16-byte activation unit per thread per stage");
    static_assert(R * U % 256 == 0, "whole units per thread");
};

constexpr int kPastEnd = 0x7ffffff0;   // an offset past every resource: reads zero

// Whole activation column in LDS when it is at most 32 KB of f16.
constexpr int64_t kWholeMaxK = 16384;

// Two f32 bit patterns rounded to f16 and packed (low element first).
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi)
{
    return (uint32_t)rne_f16(__uint_as_float(lo)) | ((uint32_t)rne_f16(__uint_as_float(hi)) << 16);
}

// Rounded f16 bit patterns of eight consecutive activation elements held as
// raw data: two 16-byte halves of f32 values (kF32), or one of f16 patterns.
// (Elements are copied out of the vectors before the bit cast: this clang
// miscompiles __builtin_bit_cast applied to a vector element in place.)
template <bool kF32>
__device__ __forceinline__ u32x4 round8(const u32x4 (&r)[2])
{
    if (!kF32) return r[0];
    const u32x4 p = r[0], q = r[1];
    u32x4 o;
    o[0] = pack2(p[0], p[1]);
    o[1] = pack2(p[2], p[3]);
    o[2] = pack2(q[0], q[1]);
    o[3] = pack2(q[2], q[3]);
    return o;
}

// kWhole: the whole activation column (k <= 16384 elements) is rounded or
// copied into LDS once at the start, overlapping the first weight stages, and
// the stages carry weights only; otherwise each stage also stages its SC
// activation elements.  Dynamic LDS: 2 * (WBYTES, or BUFB) + (k * 2 if kWhole).
//
// Every block takes R rows of one matrix (row tile blockIdx.x - tile0[m] of
// matrix m).  Weights and per-stage activations come through buffer loads
// whose resources end at the tile's last row and the column's last element:
// rows past the matrix, elements past k and stages past the last read zero
// without a branch or any memory traffic, so every stage issues the same
// loads and the compiler can wait for exactly the stage it needs.
//
// D register sets: the loads of stages s + 1 .. s + D are in flight while
// stage s is multiplied (stage s + 1 waits in its registers until it is
// copied into the other LDS buffer).  Matrices of a few thousand rows give
// each CU only two or three blocks, so one stage in flight per block leaves
// HBM latency exposed; D = 4 keeps 64 KB per block in flight.  Elements past
// k inside a stage (the next row's, or zero) land in LDS positions the
// multiply never reads: it stops at the last full 32-element step and the
// k % 32 tail is read from global memory.
//
template <int LPR>
struct Depth {
    static constexpr int D = 4;
};

//
// lds_tile is one block's work: rows r0 .. r0 + R - 1 of the matrix wm
// (rows_m x k) against the column a, results to out (out[r] for row r).
// The GEMV kernels below call it for a row tile of a RowTable matrix, or of
// one product of a ProdTable.
template <int LPR, bool kF32, bool kWhole>
__device__ __forceinline__ void lds_tile(const uint16_t *__restrict__ wm, int64_t rows_m, int64_t r0, int64_t k,
                                         const void *__restrict__ a, float *__restrict__ out)
{
    typedef LdsCfg<LPR> C;
    typedef typename Halves<C::CPL>::T HT;
    constexpr int D = Depth<LPR>::D;
    constexpr int BUF = kWhole ? C::WBYTES : C::BUFB;   // bytes per stage buffer
    constexpr int ESZ = kF32 ? 4 : 2;                    // activation element bytes
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *actl = lds + 2 * BUF;                 // whole column (kWhole)

    const int tid = threadIdx.x;
    const int64_t vrows = rows_m - r0 < C::R ? rows_m - r0 : C::R;
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wm + r0 * k, vrows * k * 2);
    const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(a, k * ESZ);

    // This thread's stage units: unit p is 16 bytes of row urow(p) at
    // element 8 * ucol(p); stage s adds 2 * SC * s.  kWhole: each wave stages
    // exactly the R / 4 rows it multiplies (rows rho = tid / LPR of its 64
    // threads), so no other wave reads what it writes and a stage needs only
    // the wave's own LDS wait, no block barrier (the shared column is in LDS
    // before the loop).  Otherwise the 256 threads split each row's units
    // and the per-stage activation, and every stage ends with a barrier.
    auto urow = [&](int p) {
        return kWhole ? (tid >> 6) * (C::R / 4) + (p * 64 + (tid & 63)) / C::U : (p * 256 + tid) / C::U;
    };
    auto ucol = [&](int p) { return kWhole ? (p * 64 + (tid & 63)) % C::U : (p * 256 + tid) % C::U; };
    int woff[C::UPT];
#pragma unroll
    for (int p = 0; p < C::UPT; p++) woff[p] = (int)(urow(p) * k * 2 + 16 * ucol(p));
    const bool act_loader = tid < C::U;
    const int aoff = act_loader ? 8 * tid * ESZ : kPastEnd;

    const int64_t nsteps = k >> 5;                       // full 32-element steps
    const int64_t nstages = (k + C::SC - 1) / C::SC;

    u32x4 wreg[D][C::UPT];
    u32x4 areg[D][2];
    auto fetch = [&](int64_t s, int set) {
        const bool live = s < nstages;
        const int so = live ? (int)(s * C::SC * 2) : 0;
#pragma unroll
        for (int p = 0; p < C::UPT; p++)
            wreg[set][p] = __builtin_amdgcn_raw_buffer_load_b128(wr, live ? woff[p] + so : kPastEnd, 0, 2);
        if (!kWhole) {
            const int ao = live && act_loader ? aoff + (int)(s * C::SC * ESZ) : kPastEnd;
            areg[set][0] = __builtin_amdgcn_raw_buffer_load_b128(ar, ao, 0, 0);
            if (kF32) areg[set][1] = __builtin_amdgcn_raw_buffer_load_b128(ar, ao == kPastEnd ? ao : ao + 16, 0, 0);
        }
    };
    auto stash = [&](int set, int buf) {
        unsigned char *base = lds + buf * BUF;
#pragma unroll
        for (int p = 0; p < C::UPT; p++)
            *reinterpret_cast<u32x4 *>(base + urow(p) * C::ROWB + 16 * ucol(p)) = wreg[set][p];
        if (!kWhole && act_loader)
            *reinterpret_cast<u32x4 *>(base + C::WBYTES + 16 * tid) = round8<kF32>(areg[set]);
    };

    const int rho = tid / LPR;
    const int j = tid % LPR;
    float acc[C::CPL];
#pragma unroll
    for (int i = 0; i < C::CPL; i++) acc[i] = 0.f;

    auto compute = [&](int64_t s) {
        const int buf = (int)(s & 1);
        const unsigned char *wl = lds + buf * BUF + rho * C::ROWB + j * C::CPL * 2;
        const unsigned char *al = kWhole ? actl + 2 * s * C::SC + j * C::CPL * 2
                                         : lds + buf * C::BUFB + C::WBYTES + j * C::CPL * 2;
        const int64_t left = nsteps - s * (C::SC / 32);
        if (left >= C::SC / 32) {
#pragma unroll 8
            for (int st = 0; st < C::SC / 32; st++)
                fma_halves<C::CPL>(acc, *reinterpret_cast<const HT *>(wl + 64 * st),
                                   *reinterpret_cast<const HT *>(al + 64 * st));
        } else {
            for (int st = 0; st < (int)left; st++)
                fma_halves<C::CPL>(acc, *reinterpret_cast<const HT *>(wl + 64 * st),
                                   *reinterpret_cast<const HT *>(al + 64 * st));
        }
    };

    // Prologue.  The whole activation column (kWhole) is loaded first, 8
    // elements per thread per round for every round a column of kWholeMaxK
    // elements needs (rounds past k read zero and move no data), so the
    // load count is the same for every k; then the first D weight stages.
    // The column is written to LDS as soon as its own loads are in, while the
    // weight stages are still in flight.
    constexpr int NAR = kWhole ? (int)(kWholeMaxK / (8 * 256)) : 1;   // rounds
    u32x4 araw[NAR][2];
    if (kWhole) {
#pragma unroll
        for (int i = 0; i < NAR; i++) {
            const int off = (tid + 256 * i) * 8 * ESZ;
            araw[i][0] = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
            if (kF32) araw[i][1] = __builtin_amdgcn_raw_buffer_load_b128(ar, off + 16, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep them ahead of the weight loads
    }
#pragma unroll
    for (int d = 0; d < D; d++) fetch(d, d);
    if (kWhole) {
        // k % 8 == 0 here; visible to every thread after the barrier below
#pragma unroll
        for (int i = 0; i < NAR; i++) {
            const int64_t e = 8 * (tid + 256 * i);
            if (e < k) *reinterpret_cast<u32x4 *>(actl + 2 * e) = round8<kF32>(araw[i]);
        }
    }
    stash(0, 0);
    __syncthreads();
    // Stage s sits in LDS buffer s % 2 and came through register set s % D.
    // The loop runs a whole number of D-stage rounds; the stages past the
    // last only load zeros and skip the multiply, so every round issues the
    // same loads.  A wave's LDS operations execute in order, so once its
    // writes of stage s + 1 are complete (lgkmcnt(0)) it may read them, and
    // its later writes into buffer s % 2 follow its reads of stage s.  With
    // rows shared between waves (not kWhole) a plain barrier follows: each
    // wave's own LDS writes are complete before it arrives, and nothing else
    // needs to drain.
    const int64_t rounds = (nstages + D - 1) / D;
    for (int64_t s0 = 0; s0 < rounds * D; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
            const int64_t s = s0 + d;
            fetch(s + D, d);                     // set d is free: stage s is in LDS
            if (s < nstages) compute(s);
            stash((d + 1) % D, (int)((s + 1) & 1));
            if (kWhole)
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            else
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    }

    float v = vec_dot_tree<C::CPL>(acc);
    const int64_t r = r0 + rho;
    if (j == 0 && r < rows_m) {
        const uint16_t *wrow = wm + r * k;
        if (k & 31) v = add_tail<kF32>(v, wrow, a, nsteps * 32, k);
        out[r] = v;
    }
}

// Row tile blockIdx.x - tile0[m] of matrix m of the RowTable, against column
// blockIdx.y.
template <int LPR, bool kF32, bool kWhole>
__global__ __launch_bounds__(256) void vec_dot_lds(RowTable t, int64_t k, const void *__restrict__ a_all)
{
    constexpr int ESZ = kF32 ? 4 : 2;
    const int64_t col = blockIdx.y;
    int m = 0;
#pragma unroll
    for (int i = 1; i < F16WM_MAX_MULTI; i++)
        if (i < t.count && (int64_t)blockIdx.x >= t.tile0[i]) m = i;
    const int64_t rows_m = t.row0[m + 1] - t.row0[m];
    const int64_t r0 = ((int64_t)blockIdx.x - t.tile0[m]) * LdsCfg<LPR>::R;
    lds_tile<LPR, kF32, kWhole>(t.w[m], rows_m, r0, k, static_cast<const char *>(a_all) + col * k * ESZ,
                                t.out[m] + col * rows_m);
}

// The product of a ProdTable that block b belongs to: the last p with
// tile0[p] <= b (binary search over the table in the kernel arguments).
__device__ __forceinline__ int table_product(const ProdTable &t, int b)
{
    int lo = 0, hi = t.count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t.tile0[mid] <= b) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Row tile blockIdx.x - tile0[p] of product p of the table (each product
// has its own weight, column, k and output).
template <int LPR, bool kF32, bool kWhole>
__global__ __launch_bounds__(256) void vec_dot_lds_table(ProdTable t)
{
    const int p = table_product(t, (int)blockIdx.x);
    const int64_t r0 = (int64_t)((int)blockIdx.x - t.tile0[p]) * LdsCfg<LPR>::R;
    lds_tile<LPR, kF32, kWhole>(t.w[p], t.rows[p], r0, t.k[p], t.a[p], t.out[p]);
}

// Short rows (k <= kDirectMaxK, k % 8 == 0, 16-byte aligned): no staging.
// A one-wave block takes 16 consecutive rows of one matrix, four lanes per
// row, lane j owning chains 8j .. 8j + 7 (the 8 elements of one 16-byte
// piece of each step).  Every load is issued up front: first the activation
// column, then every weight step of the row, straight into registers, so the
// whole row arrives in one memory round trip and the column is rounded into
// LDS while the weights are still in flight.  Chains, tree, tail and store as
// in vec_dot_lds.  For the many small matrices of a small model's decode step,
// where a launch is a few round trips long.
constexpr int kDirectMaxK = 576;              // 18 steps of 32
constexpr int kDirectRows = 16;               // rows per one-wave block
static_assert(kDirectMaxK == kDirectMaxKTable && kDirectRows == kTableRowsDirect, "table launcher's view");
static_assert(LdsCfg<16>::R == kTableRowsLds, "table launcher's view");

// direct_tile: rows 0 .. vrows - 1 of w0 (a matrix with k columns, from its
// row r0), lane quad q = threadIdx.x / 4 taking row q, against the column a;
// row q's result to dst[q].  The loads go through buffer resources that end
// at the tile's last row and the column's last element, and steps past k
// read from past the end: all of them read zero without memory traffic, so
// every lane issues the same loads with no branch, and the wait for the
// column (issued first) leaves the weight loads in flight.  The block's 64
// threads share `actl` (kDirectMaxK halves of LDS) for the rounded column.
template <bool kF32>
__device__ __forceinline__ void direct_tile(unsigned char *actl, const uint16_t *__restrict__ w0, int vrows,
                                            int64_t k, const void *__restrict__ a, float *__restrict__ dst)
{
    constexpr int MAXS = kDirectMaxK / 32;
    constexpr int ESZ = kF32 ? 4 : 2;
    constexpr int NR = (kDirectMaxK / 8 + 63) / 64;   // column rounds of 64 threads x 8 elements
    const int tid = threadIdx.x;
    const int q = tid >> 2, j = tid & 3;
    const int nsteps = (int)(k >> 5);
    const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(a, k * ESZ);
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(w0, vrows * k * 2);

    u32x4 raw[NR][2];
#pragma unroll
    for (int r = 0; r < NR; r++) {
        const int off = (64 * r + tid) * 8 * ESZ;
        raw[r][0] = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
        if (kF32) raw[r][1] = __builtin_amdgcn_raw_buffer_load_b128(ar, off + 16, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep them ahead of the weight loads
    const int wbase = (int)(q * k * 2) + 16 * j;
    u32x4 wv[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; s++)
        wv[s] = __builtin_amdgcn_raw_buffer_load_b128(wr, s < nsteps ? wbase + 64 * s : kPastEnd, 0, 2);
    // the column, rounded, 8 elements per thread and round (k % 8 == 0)
#pragma unroll
    for (int r = 0; r < NR; r++) {
        const int u = 64 * r + tid;
        if (8 * u < k) *reinterpret_cast<u32x4 *>(actl + 16 * u) = round8<kF32>(raw[r]);
    }
    __syncthreads();

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < MAXS; s++)
        if (s < nsteps) fma_halves<8>(acc, wv[s], *reinterpret_cast<const u32x4 *>(actl + 64 * s + 16 * j));
    float v = vec_dot_tree<8>(acc);
    if (q < vrows && j == 0) {
        if (k & 31) v = add_tail<kF32>(v, w0 + q * k, a, (int64_t)nsteps * 32, k);
        dst[q] = v;
    }
}

// Row tile blockIdx.x - tile0[m] of matrix m of the RowTable (16 rows of one
// matrix), column blockIdx.y.
template <bool kF32>
__global__ __launch_bounds__(64) void vec_dot_direct(RowTable t, int64_t k, const void *__restrict__ a_all)
{
    __shared__ __attribute__((aligned(16))) unsigned char actl[kDirectMaxK * 2];
    const int64_t col = blockIdx.y;
    int m = 0;
#pragma unroll
    for (int i = 1; i < F16WM_MAX_MULTI; i++)
        if (i < t.count && (int64_t)blockIdx.x >= t.tile0[i]) m = i;
    const int64_t rows_m = t.row0[m + 1] - t.row0[m];
    const int64_t r0 = ((int64_t)blockIdx.x - t.tile0[m]) * kDirectRows;
    const int vrows = (int)(rows_m - r0 < kDirectRows ? rows_m - r0 : kDirectRows);
    direct_tile<kF32>(actl, t.w[m] + r0 * k, vrows, k, static_cast<const char *>(a_all) + col * k * (kF32 ? 4 : 2),
                      t.out[m] + col * rows_m + r0);
}

// Rows 16 (blockIdx.x - tile0[p]) .. + 15 of product p of the table.
template <bool kF32>
__global__ __launch_bounds__(64) void vec_dot_direct_table(ProdTable t)
{
    __shared__ __attribute__((aligned(16))) unsigned char actl[kDirectMaxK * 2];
    const int p = table_product(t, (int)blockIdx.x);
    const int64_t k = t.k[p];
    const int64_t r0 = (int64_t)((int)blockIdx.x - t.tile0[p]) * kDirectRows;
    const int vrows = (int)(t.rows[p] - r0 < kDirectRows ? t.rows[p] - r0 : kDirectRows);
    direct_tile<kF32>(actl, t.w[p] + r0 * k, vrows, k, t.a[p], t.out[p] + r0);
}

constexpr int kV1Rows = 8;    // rows per 256-thread block, 32 lanes per row

template <bool kF32>
__global__ __launch_bounds__(256) void vec_dot_v1(RowTable t, int64_t k, const void *__restrict__ a_all)
{
    const int64_t col = blockIdx.y;
    const void *a = static_cast<const char *>(a_all) + col * k * (kF32 ? 4 : 2);
    const int c = threadIdx.x & 31;
    const int64_t g = (int64_t)blockIdx.x * kV1Rows + (threadIdx.x >> 5);
    const bool valid = g < t.row0[t.count];
    const int m = find_matrix(t, valid ? g : 0);
    const int64_t r = valid ? g - t.row0[m] : 0;
    const uint16_t *wrow = t.w[m] + r * k;
    const int64_t nsteps = k >> 5;

    float acc = 0.f;
    if (valid) {
#pragma unroll 8
        for (int64_t s = 0; s < nsteps; s++)
            acc = __builtin_fmaf(widen(wrow[32 * s + c]), widen(act16<kF32>(a, 32 * s + c)), acc);
    }
    acc = acc + __shfl_xor(acc, 16);   // a0 + a2, a1 + a3
    acc = acc + __shfl_xor(acc, 8);    // (a0 + a2) + (a1 + a3)
    acc = acc + __shfl_xor(acc, 4);    // low half + high half
    acc = acc + __shfl_xor(acc, 1);    // horizontal add: adjacent pairs
    acc = acc + __shfl_xor(acc, 2);    // horizontal add: the two pair sums

    if (valid && c == 0) {
        float v = acc;
        if (k & 31) v = add_tail<kF32>(v, wrow, a, nsteps * 32, k);
        const int64_t rows_m = t.row0[m + 1] - t.row0[m];
        t.out[m][col * rows_m + r] = v;
    }
}


// Launches one instantiation with its dynamic LDS allowed first.
template <typename K>
void launch_with_lds(K kernel, int max_bytes, dim3 grid, size_t shm, hipStream_t stream, const RowTable &t,
                     int64_t k, const void *a)
{
    allow_dynamic_lds(reinterpret_cast<const void *>(kernel), max_bytes);
    kernel<<<grid, dim3(256), shm, stream>>>(t, k, a);
}

template <int LPR>
void launch_lds(dim3 grid, hipStream_t stream, const RowTable &t, int64_t k, const void *a, bool f32act)
{
    typedef LdsCfg<LPR> C;
    if (k <= kWholeMaxK) {
        const int max_shm = 2 * C::WBYTES + (int)kWholeMaxK * 2;
        const size_t shm = 2 * C::WBYTES + (size_t)k * 2;
        if (f32act)
            launch_with_lds(vec_dot_lds<LPR, true, true>, max_shm, grid, shm, stream, t, k, a);
        else
            launch_with_lds(vec_dot_lds<LPR, false, true>, max_shm, grid, shm, stream, t, k, a);
    } else {
        const int shm = 2 * C::BUFB;
        if (f32act)
            launch_with_lds(vec_dot_lds<LPR, true, false>, shm, grid, shm, stream, t, k, a);
        else
            launch_with_lds(vec_dot_lds<LPR, false, false>, shm, grid, shm, stream, t, k, a);
    }
}

template <bool kF32, bool kWhole>
hipError_t launch_lds_table(const ProdTable &t, int64_t maxk, hipStream_t stream)
{
    typedef LdsCfg<16> C;
    const int max_shm = kWhole ? 2 * C::WBYTES + (int)kWholeMaxK * 2 : 2 * C::BUFB;
    const size_t shm = kWhole ? 2 * C::WBYTES + (size_t)maxk * 2 : 2 * C::BUFB;
    allow_dynamic_lds(reinterpret_cast<const void *>(vec_dot_lds_table<16, kF32, kWhole>), max_shm);
    vec_dot_lds_table<16, kF32, kWhole><<<dim3((uint32_t)t.tile0[t.count]), dim3(256), shm, stream>>>(t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_vec_dot_table(ProdTable t, bool direct, bool f32act, hipStream_t stream)
{
    const int per = direct ? kDirectRows : LdsCfg<16>::R;
    int64_t tiles = 0, maxk = 0;
    for (int p = 0; p < t.count; p++) {
        t.tile0[p] = (int32_t)tiles;
        tiles += ((int64_t)t.rows[p] + per - 1) / per;
        if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
        if (t.k[p] > maxk) maxk = t.k[p];
    }
    t.tile0[t.count] = (int32_t)tiles;
    if (tiles == 0) return hipSuccess;
    if (direct) {
        if (maxk > kDirectMaxK) return hipErrorInvalidValue;
        if (f32act)
            vec_dot_direct_table<true><<<dim3((uint32_t)tiles), dim3(64), 0, stream>>>(t);
        else
            vec_dot_direct_table<false><<<dim3((uint32_t)tiles), dim3(64), 0, stream>>>(t);
        return hipGetLastError();
    }
    if (maxk <= kWholeMaxK)
        return f32act ? launch_lds_table<true, true>(t, maxk, stream) : launch_lds_table<false, true>(t, maxk, stream);
    return f32act ? launch_lds_table<true, false>(t, maxk, stream) : launch_lds_table<false, false>(t, maxk, stream);
}

hipError_t launch_vec_dot(const RowTable &t, int64_t k, const void *a, bool f32act, int64_t ncols,
                          bool vec8, hipStream_t stream)
{
    const int64_t total = t.row0[t.count];
    // Lanes per row: 16 from 4096 rows on, else 32 (measured on the 8B
    // shapes: 16 lanes beat 32 by 5-15 % on the 4096- and 6144-row products
    // and 64-row blocks with 4 lanes by 3 % on the 128256-row logits; 8 lanes
    // per row was never faster).
    const int lpr = vec8 && total >= 4096 ? 16 : 32;
    if (vec8 && k <= kDirectMaxK) {
        RowTable td = t;
        int64_t bx = 0;
        for (int i = 0; i < t.count; i++) {
            td.tile0[i] = bx;
            bx += (t.row0[i + 1] - t.row0[i] + kDirectRows - 1) / kDirectRows;
        }
        td.tile0[t.count] = bx;
        if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;
        for (int64_t c0 = 0; c0 < ncols; c0 += 65535) {
            const int64_t nc = ncols - c0 < 65535 ? ncols - c0 : 65535;
            RowTable tc = td;
            for (int i = 0; i < t.count; i++) tc.out[i] = t.out[i] + c0 * (t.row0[i + 1] - t.row0[i]);
            const void *ac = static_cast<const char *>(a) + c0 * k * (f32act ? 4 : 2);
            if (f32act)
                vec_dot_direct<true><<<dim3((uint32_t)bx, (uint32_t)nc), dim3(64), 0, stream>>>(tc, k, ac);
            else
                vec_dot_direct<false><<<dim3((uint32_t)bx, (uint32_t)nc), dim3(64), 0, stream>>>(tc, k, ac);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // The LDS kernels address one row tile through 32-bit buffer offsets.
    if (vec8 && (256 / 16) * k * 2 + 65536 > 0x7fff0000) vec8 = false;
    const int per = vec8 ? 256 / lpr : kV1Rows;
    RowTable tt = t;
    int64_t bx = (total + per - 1) / per;
    if (vec8) {
        bx = 0;
        for (int i = 0; i < t.count; i++) {
            tt.tile0[i] = bx;
            bx += (t.row0[i + 1] - t.row0[i] + per - 1) / per;
        }
        tt.tile0[t.count] = bx;
    }
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    // grid.y is limited to 65535: launch column chunks, each with its own
    // activation and output offsets.
    for (int64_t c0 = 0; c0 < ncols; c0 += 65535) {
        const int64_t nc = ncols - c0 < 65535 ? ncols - c0 : 65535;
        RowTable tc = tt;
        for (int i = 0; i < t.count; i++) tc.out[i] = t.out[i] + c0 * (t.row0[i + 1] - t.row0[i]);
        const dim3 grid((uint32_t)bx, (uint32_t)nc);
        const void *ac = static_cast<const char *>(a) + c0 * k * (f32act ? 4 : 2);
        if (!vec8) {
            if (f32act)
                vec_dot_v1<true><<<grid, dim3(256), 0, stream>>>(tc, k, ac);
            else
                vec_dot_v1<false><<<grid, dim3(256), 0, stream>>>(tc, k, ac);
        } else if (lpr == 16) {
            launch_lds<16>(grid, stream, tc, k, ac, f32act);
        } else {
            launch_lds<32>(grid, stream, tc, k, ac, f32act);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace f16wm
