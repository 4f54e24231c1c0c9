// tinyBLAS order on gfx950: the exact product for n >= 2 columns when
// rows % 4 == 0 and k % 8 == 0.
//
// bankML f16 page, Design notes ("sgemm_dot" and "Blocking"): every output
// element is ONE chain of eight f32 lanes, lane l taking elements 8t + l in
// ascending t, each step an FMA; the element is then reduced
// ((l0 + l4) + (l2 + l6)) + ((l1 + l5) + (l3 + l7)).  Register blocking decides
// who computes an element, never its bits.  Matrix products (mat_mul_par):
// out[c*rows + r]; the activation columns are widened once per product.
//
// gfx950 design (VALU fp32 FMAs; the order rules out the matrix cores):
//  - The eight chain lanes of an element are split over four threads: thread
//    q of an element group owns lanes q and q + 4.  The hsum then starts
//    in-thread ((l_q + l_{q+4})) and finishes with a shuffle between q and
//    q ^ 2 ((l0+l4) + (l2+l6) and (l1+l5) + (l3+l7)) and one between q and
//    q ^ 1: the page's tree exactly.
//  - A 256-thread block owns a 64-row x 64-column output tile; each thread
//    owns 8 rows x 8 columns x its 2 lanes = 128 accumulators.
//  - Each 64-element k stage is loaded from global memory as f16, widened
//    exactly to f32 once and stored in LDS as, for every lane pair q and
//    every pair of steps, the four values (x[8t+q], x[8t+q+4], x[8t+8+q],
//    x[8t+8+q+4]): one 16-byte LDS read feeds 16 FMAs of a thread (two
//    steps of both its lanes for one row or column).  The FMAs are plain
//    v_fma_f32 (full rate; the f16-operand form runs at two thirds of it).
//  - Stages past k are zero (loads beyond the row read nothing): a chain
//    step adding fma(0, 0, acc) = acc + 0 leaves every accumulator
//    unchanged, because an accumulator that starts at +0 never becomes -0.
//  - Blocks walk the output tiles in an XCD-aware order (block b runs on
//    XCD b % 8, each XCD takes a contiguous range of tiles, the column tiles
//    of one weight-row block are consecutive), so each weight row block is
//    read from HBM once and re-read from that XCD's L2.
//
// ALU-bound: rows*n*k FMAs.
#include "kernels.h"

namespace f16wm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 64;              // weight rows per block
constexpr int kBN = 64;              // activation columns per block
constexpr int kKS = 64;              // k per stage: 8 chain steps
constexpr int kTP = kKS / 16;        // step pairs per stage
constexpr int kQS = kTP * 64 + 4;    // f32x4 slots between lane-pair groups (4 KB + 64 B)
constexpr int kOp = 4 * kQS;         // f32x4 slots of one operand per buffer

template <bool kAligned>
__device__ __forceinline__ u32x4 load8(const uint16_t *p)
{
    if (kAligned) return *reinterpret_cast<const u32x4 *>(p);
    u32x4 v;
    v.x = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
    v.y = (uint32_t)p[2] | ((uint32_t)p[3] << 16);
    v.z = (uint32_t)p[4] | ((uint32_t)p[5] << 16);
    v.w = (uint32_t)p[6] | ((uint32_t)p[7] << 16);
    return v;
}

// Global -> registers for one stage: 2 weight and 2 activation 8-element units
// per thread (unit idx: row idx >> 3, step idx & 7), zero past rows, n or k.
template <bool kAligned>
__device__ __forceinline__ void fetch_stage(u32x4 (&wreg)[2], u32x4 (&areg)[2], const uint16_t *w,
                                            int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                                            int64_t row0, int64_t col0, int64_t k0, int tid)
{
#pragma unroll
    for (int p = 0; p < 2; p++) {
        const int idx = p * 256 + tid;
        const int rr = idx >> 3;
        const int64_t gk = k0 + 8 * (idx & 7);
        const int64_t gr = row0 + rr, gc = col0 + rr;
        u32x4 wv = {0u, 0u, 0u, 0u}, av = {0u, 0u, 0u, 0u};
        if (gr < rows && gk < k) wv = load8<kAligned>(w + gr * k + gk);
        if (gc < n && gk < k) av = load8<kAligned>(a + gc * k + gk);
        wreg[p] = wv;
        areg[p] = av;
    }
}

// Widen one 8-element unit (row r, step t of the stage) and store its four
// lane pairs: pair q goes to slot [q][t / 2][r], half (t % 2).
__device__ __forceinline__ void stash_unit(f32x4 *op, u32x4 v, int r, int t)
{
    const half8 h = __builtin_bit_cast(half8, v);
    float *base = reinterpret_cast<float *>(op + (t >> 1) * 64 + r) + 2 * (t & 1);
#pragma unroll
    for (int q = 0; q < 4; q++) {
        f32x2 pr;
        pr.x = (float)h[q];
        pr.y = (float)h[q + 4];
        *reinterpret_cast<f32x2 *>(base + q * kQS * 4) = pr;
    }
}

template <bool kAligned>
__global__ __launch_bounds__(256) void sgemm_kernel(GemmTable g, int64_t k, const uint16_t *__restrict__ a,
                                                    int64_t n, int nct)
{
    __shared__ f32x4 lds[2][2 * kOp];    // [buffer][weights | activations]

    // XCD-aware tile index, then this tile's matrix
    int mi, rt, ct;
    gemm_tile(g, xcd_tile(blockIdx.x, g.tile0[g.count]), nct, mi, rt, ct);
    const uint16_t *__restrict__ w = g.w[mi];
    const int64_t rows = g.rows[mi];
    float *__restrict__ out = g.out[mi];
    const int64_t row0 = (int64_t)rt * kBM;
    const int64_t col0 = (int64_t)ct * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane & 3;                         // lanes q and q + 4 of every element
    const int o = lane >> 2;                        // element group within the wave (4 x 4)
    const int orow = (wave >> 1) * 4 + (o >> 2);    // rows orow + 8 i
    const int ocol = (wave & 1) * 4 + (o & 3);      // columns ocol + 8 j

    float acc[8][8][2];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j][0] = acc[i][j][1] = 0.f;

    const int64_t nstages = (k + kKS - 1) / kKS;
    u32x4 wreg[2], areg[2];
    if (nstages > 0) fetch_stage<kAligned>(wreg, areg, w, rows, k, a, n, row0, col0, 0, tid);
    for (int64_t s = 0; s < nstages; s++) {
        const int buf = (int)(s & 1);
        f32x4 *wl = lds[buf];
        f32x4 *al = lds[buf] + kOp;
        // Buffer buf was last read two stages ago; the barrier of the previous
        // stage separates those reads from these writes.
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const int idx = p * 256 + tid;
            stash_unit(wl, wreg[p], idx >> 3, idx & 7);
            stash_unit(al, areg[p], idx >> 3, idx & 7);
        }
        __syncthreads();
        if (s + 1 < nstages)
            fetch_stage<kAligned>(wreg, areg, w, rows, k, a, n, row0, col0, (s + 1) * kKS, tid);
        const f32x4 *wq = wl + q * kQS;
        const f32x4 *aq = al + q * kQS;
#pragma unroll
        for (int tp = 0; tp < kTP; tp++) {
            f32x4 wv[8], av[8];
#pragma unroll
            for (int i = 0; i < 8; i++) wv[i] = wq[tp * 64 + orow + 8 * i];
#pragma unroll
            for (int j = 0; j < 8; j++) av[j] = aq[tp * 64 + ocol + 8 * j];
            // step 2 tp, then step 2 tp + 1, for lanes q (x, z) and q + 4 (y, w)
#pragma unroll
            for (int i = 0; i < 8; i++)
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    acc[i][j][0] = __builtin_fmaf(wv[i].x, av[j].x, acc[i][j][0]);
                    acc[i][j][1] = __builtin_fmaf(wv[i].y, av[j].y, acc[i][j][1]);
                }
#pragma unroll
            for (int i = 0; i < 8; i++)
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    acc[i][j][0] = __builtin_fmaf(wv[i].z, av[j].z, acc[i][j][0]);
                    acc[i][j][1] = __builtin_fmaf(wv[i].w, av[j].w, acc[i][j][1]);
                }
        }
    }

    // hsum: (l_q + l_{q+4}) in-thread, then with q ^ 2, then with q ^ 1.
    // Every lane of the group ends with the element; lane q stores the
    // columns j with j % 4 == q.
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t r = row0 + orow + 8 * i;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float v = acc[i][j][0] + acc[i][j][1];
            v = v + __shfl_xor(v, 2);
            v = v + __shfl_xor(v, 1);
            const int64_t c = col0 + ocol + 8 * j;
            if ((j & 3) == q && r < rows && c < n) out[c * rows + r] = v;
        }
    }
}

}  // namespace

hipError_t launch_sgemm(GemmTable g, int64_t k, const uint16_t *a, int64_t n, bool aligned16,
                        hipStream_t stream)
{
    const int64_t nct = (n + kBN - 1) / kBN;
    int64_t tiles = 0;
    for (int i = 0; i < g.count; i++) {
        g.tile0[i] = (int32_t)tiles;
        tiles += (g.rows[i] + kBM - 1) / kBM * nct;
        if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    }
    g.tile0[g.count] = (int32_t)tiles;
    const dim3 grid((uint32_t)tiles);
    if (aligned16)
        sgemm_kernel<true><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    else
        sgemm_kernel<false><<<grid, dim3(256), 0, stream>>>(g, k, a, n, (int)nct);
    return hipGetLastError();
}

}  // namespace f16wm
