// tinyBLAS order on gfx950: the exact product for n >= 2 columns when
// rows % 4 == 0 and k % 8 == 0.
//
// bankML f16 page, Design notes ("sgemm_dot" and "Blocking"): every output
// element is ONE chain of eight f32 lanes, lane l taking elements 8t + l in
// ascending t, each step an FMA; the element is then reduced
// ((l0 + l4) + (l2 + l6)) + ((l1 + l5) + (l3 + l7)).  Register blocking decides
// who computes an element, never its bits.  Matrix products (mat_mul_par):
// out[c*rows + r].
//
// gfx950 design: VALU fp32 FMAs (the order forbids the matrix cores).  A
// 256-thread block owns a 64-row x 64-column tile of outputs; each thread owns
// 4 rows x 4 columns x all 8 chain lanes = 128 accumulators, so the final
// reduction is in-register.  Per step t of 8 elements a thread reads four
// 16-byte weight vectors and four 16-byte activation vectors from LDS and
// issues 128 FMAs whose f16 operands are widened exactly by v_fma_mix_f32.
// Tiles are staged global -> registers -> LDS, with the next stage's global
// loads in flight while the current stage computes.
//
// ALU-bound: rows*n*k FMAs; each weight byte is re-read n/64 times and each
// activation byte rows/64 times, from L2.
#include "kernels.h"

namespace f16wm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;    // weight rows per block
constexpr int kBN = 64;    // activation columns per block
constexpr int kBKV = 8;    // 8-element k vectors per stage (64 elements)

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

// Global -> registers for one stage: 2 weight and 2 activation vectors.
template <bool kAligned>
__device__ __forceinline__ void fetch_stage(u32x4 (&wreg)[2], u32x4 (&areg)[2], const uint16_t *w,
                                            int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                                            int64_t row0, int64_t col0, int64_t kv0, int64_t kvs,
                                            int tid)
{
#pragma unroll
    for (int p = 0; p < 2; p++) {
        const int idx = tid + 256 * p;
        const int rr = idx >> 3, kk = idx & 7;
        const int64_t gk = kv0 + kk;
        const int64_t gr = row0 + rr, gc = col0 + rr;
        u32x4 wv = {0u, 0u, 0u, 0u}, av = {0u, 0u, 0u, 0u};
        if (gr < rows && gk < kvs) wv = load8<kAligned>(w + gr * k + gk * 8);
        if (gc < n && gk < kvs) av = load8<kAligned>(a + gc * k + gk * 8);
        wreg[p] = wv;
        areg[p] = av;
    }
}

// Operands of one step t (8 elements): the thread's 4 weight vectors and 4
// activation vectors.
struct StepRegs {
    u32x4 w[4], a[4];
};

__device__ __forceinline__ void read_step(StepRegs &r, const u32x4 (*Ws)[kBM], const u32x4 (*As)[kBN],
                                          int s, int tx, int ty)
{
#pragma unroll
    for (int i = 0; i < 4; i++) r.w[i] = Ws[s][tx + 16 * i];
#pragma unroll
    for (int j = 0; j < 4; j++) r.a[j] = As[s][ty + 16 * j];
}

// One chain step for the thread's 4 x 4 elements x 8 chain lanes.
__device__ __forceinline__ void chain_step(float (&acc)[4][4][8], const StepRegs &r)
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const half8 wh = __builtin_bit_cast(half8, r.w[i]);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const half8 ah = __builtin_bit_cast(half8, r.a[j]);
#pragma unroll
            for (int l = 0; l < 8; l++)
                acc[i][j][l] = __builtin_fmaf((float)wh[l], (float)ah[l], acc[i][j][l]);
        }
    }
}

template <bool kAligned>
__global__ __launch_bounds__(256) void sgemm_kernel(const uint16_t *__restrict__ w, int64_t rows,
                                                    int64_t k, const uint16_t *__restrict__ a,
                                                    int64_t n, float *__restrict__ out)
{
    __shared__ u32x4 Ws[kBKV][kBM];
    __shared__ u32x4 As[kBKV][kBN];

    const int tid = threadIdx.x;
    const int tx = tid & 15;          // rows tx + 16 i
    const int ty = tid >> 4;          // columns ty + 16 j
    const int64_t row0 = (int64_t)blockIdx.x * kBM;
    const int64_t col0 = (int64_t)blockIdx.y * kBN;
    const int64_t kvs = k >> 3;       // 8-element vectors per row

    float acc[4][4][8];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int l = 0; l < 8; l++) acc[i][j][l] = 0.f;

    u32x4 wreg[2], areg[2];
    if (kvs > 0) fetch_stage<kAligned>(wreg, areg, w, rows, k, a, n, row0, col0, 0, kvs, tid);
    for (int64_t kv0 = 0; kv0 < kvs; kv0 += kBKV) {
        __syncthreads();   // every thread is done reading the previous stage
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const int idx = tid + 256 * p;
            Ws[idx & 7][idx >> 3] = wreg[p];
            As[idx & 7][idx >> 3] = areg[p];
        }
        __syncthreads();
        if (kv0 + kBKV < kvs)
            fetch_stage<kAligned>(wreg, areg, w, rows, k, a, n, row0, col0, kv0 + kBKV, kvs, tid);
        const int64_t left = kvs - kv0;
        if (left >= kBKV) {
            // operands of step s + 1 are read from LDS while step s computes
            StepRegs r0, r1;
            read_step(r0, Ws, As, 0, tx, ty);
#pragma unroll
            for (int s2 = 0; s2 < kBKV; s2 += 2) {
                read_step(r1, Ws, As, s2 + 1, tx, ty);
                chain_step(acc, r0);
                if (s2 + 2 < kBKV) read_step(r0, Ws, As, s2 + 2, tx, ty);
                chain_step(acc, r1);
            }
        } else {
            for (int s2 = 0; s2 < (int)left; s2++) {
                StepRegs r;
                read_step(r, Ws, As, s2, tx, ty);
                chain_step(acc, r);
            }
        }
    }

#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t r = row0 + tx + 16 * i;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t c = col0 + ty + 16 * j;
            const float v = ((acc[i][j][0] + acc[i][j][4]) + (acc[i][j][2] + acc[i][j][6])) +
                            ((acc[i][j][1] + acc[i][j][5]) + (acc[i][j][3] + acc[i][j][7]));
            if (r < rows && c < n) out[c * rows + r] = v;
        }
    }
}

}  // namespace

hipError_t launch_sgemm(const uint16_t *w, int64_t rows, int64_t k, const uint16_t *a, int64_t n,
                        float *out, bool aligned16, hipStream_t stream)
{
    const int64_t bx = (rows + kBM - 1) / kBM;
    const int64_t by_all = (n + kBN - 1) / kBN;
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    for (int64_t b0 = 0; b0 < by_all; b0 += 65535) {
        const int64_t by = by_all - b0 < 65535 ? by_all - b0 : 65535;
        const int64_t c0 = b0 * kBN;
        const int64_t nc = n - c0 < by * kBN ? n - c0 : by * kBN;
        const dim3 grid((uint32_t)bx, (uint32_t)by);
        if (aligned16)
            sgemm_kernel<true><<<grid, dim3(256), 0, stream>>>(w, rows, k, a + c0 * k, nc, out + c0 * rows);
        else
            sgemm_kernel<false><<<grid, dim3(256), 0, stream>>>(w, rows, k, a + c0 * k, nc, out + c0 * rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace f16wm
