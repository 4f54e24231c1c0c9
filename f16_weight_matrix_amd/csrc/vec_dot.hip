// vec_dot order on gfx950: GEMV (one column), grouped GEMV, and the fallback
// product for shapes that do not take the tinyBLAS path.
//
// bankML f16 page, Design notes ("vec_dot"): every output element is four
// 8-lane f32 accumulators fed by FMAs over 32-element steps (accumulator j,
// lane l takes elements 32t + 8j + l, ascending t), reduced (a0+a2)+(a1+a3) lane
// by lane, then low four lanes + high four, then two horizontal adds of
// adjacent pairs; the k % 32 tail is added to that f32 in binary64 and the
// double is rounded to f32.  Matrix products (mat_vec_par,
// mat_vec_multi_par): out[r] = vec_dot(W[r], a), several matrices in one pass.
//
// Each of the 32 chains of an element is a sequential FMA chain, so one chain
// lives in one GPU lane for the whole row; the tree is a fixed sequence of
// cross-lane adds.  Both layouts below hold the same 32 chains and apply the
// same adds, so they give the same bits:
//   vec8: 4 lanes per row, lane q owns chains 8q..8q+7 and loads the 16 bytes
//         W[r][32t + 8q .. +7] per step (needs k % 8 == 0, 16-byte alignment).
//         Tree: lane q + lane q^2 is (a0+a2) / (a1+a3); then lane q + lane q^1;
//         the low/high and horizontal adds run in-lane.
//   vec1: 32 lanes per row, lane c owns chain c and loads element 32t + c.
//         Tree: lane offsets 16, 8 ((a0+a2)+(a1+a3)), 4 (low+high), 1, 2
//         (horizontal adds).
// The products of two f16 values are exact in f32, so each chain step's FMA
// equals an exact product added with one rounding; the widening of f16 inputs
// is exact (v_cvt_f32_f16 / the f16 operands of v_fma_mix_f32, with f16
// subnormals kept).
//
// HBM-bound: 2*k bytes of weight per row, read once, with the activation
// column (2*k bytes) served from cache.
#include "kernels.h"

namespace f16wm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float widen(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ void fma8(float (&acc)[8], u32x4 w, u32x4 a)
{
    const half8 wh = __builtin_bit_cast(half8, w);
    const half8 ah = __builtin_bit_cast(half8, a);
#pragma unroll
    for (int l = 0; l < 8; l++) acc[l] = __builtin_fmaf((float)wh[l], (float)ah[l], acc[l]);
}

__device__ __forceinline__ int find_matrix(const RowTable &t, int64_t g)
{
    int m = 0;
#pragma unroll
    for (int i = 1; i < F16WM_MAX_MULTI; i++)
        if (i < t.count && g >= t.row0[i]) m = i;
    return m;
}

// The k % 32 tail in binary64, ascending, onto the f32 tree result.
__device__ __forceinline__ float add_tail(float v, const uint16_t *w, const uint16_t *a, int64_t from,
                                          int64_t k)
{
    double d = (double)v;
    for (int64_t i = from; i < k; i++) {
        const float p = widen(w[i]) * widen(a[i]);   // exact in f32
        d = d + (double)p;
    }
    return (float)d;
}

constexpr int kV8Rows = 64;   // rows per 256-thread block, 4 lanes per row
constexpr int kV8Batch = 8;   // 32-element steps loaded ahead of their FMAs

__global__ __launch_bounds__(256) void vec_dot_v8(RowTable t, int64_t k,
                                                  const uint16_t *__restrict__ a_all)
{
    const int64_t col = blockIdx.y;
    const uint16_t *a = a_all + col * k;
    const int q = threadIdx.x & 3;
    const int64_t g = (int64_t)blockIdx.x * kV8Rows + (threadIdx.x >> 2);
    const bool valid = g < t.row0[t.count];
    const int m = find_matrix(t, valid ? g : 0);
    const int64_t r = valid ? g - t.row0[m] : 0;
    const uint16_t *wrow = t.w[m] + r * k;
    const int64_t nsteps = k >> 5;

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (valid) {
        const u32x4 *wp = reinterpret_cast<const u32x4 *>(wrow) + q;
        const u32x4 *ap = reinterpret_cast<const u32x4 *>(a) + q;
        int64_t s = 0;
        for (; s + kV8Batch <= nsteps; s += kV8Batch) {
            u32x4 wv[kV8Batch], av[kV8Batch];
#pragma unroll
            for (int u = 0; u < kV8Batch; u++) {
                wv[u] = __builtin_nontemporal_load(wp + 4 * (s + u));
                av[u] = ap[4 * (s + u)];
            }
#pragma unroll
            for (int u = 0; u < kV8Batch; u++) fma8(acc, wv[u], av[u]);
        }
        for (; s < nsteps; s++) fma8(acc, __builtin_nontemporal_load(wp + 4 * s), ap[4 * s]);
    }
    // (a0 + a2) and (a1 + a3), then their sum: partners q^2, then q^1.
#pragma unroll
    for (int l = 0; l < 8; l++) acc[l] = acc[l] + __shfl_xor(acc[l], 2);
#pragma unroll
    for (int l = 0; l < 8; l++) acc[l] = acc[l] + __shfl_xor(acc[l], 1);

    if (valid && q == 0) {
        const float u0 = acc[0] + acc[4], u1 = acc[1] + acc[5];   // low + high half
        const float u2 = acc[2] + acc[6], u3 = acc[3] + acc[7];
        float v = (u0 + u1) + (u2 + u3);                          // two horizontal adds
        if (k & 31) v = add_tail(v, wrow, a, nsteps * 32, k);
        const int64_t rows_m = t.row0[m + 1] - t.row0[m];
        t.out[m][col * rows_m + r] = v;
    }
}

constexpr int kV1Rows = 8;    // rows per 256-thread block, 32 lanes per row

__global__ __launch_bounds__(256) void vec_dot_v1(RowTable t, int64_t k,
                                                  const uint16_t *__restrict__ a_all)
{
    const int64_t col = blockIdx.y;
    const uint16_t *a = a_all + col * k;
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
            acc = __builtin_fmaf(widen(wrow[32 * s + c]), widen(a[32 * s + c]), acc);
    }
    acc = acc + __shfl_xor(acc, 16);   // a0 + a2, a1 + a3
    acc = acc + __shfl_xor(acc, 8);    // (a0 + a2) + (a1 + a3)
    acc = acc + __shfl_xor(acc, 4);    // low half + high half
    acc = acc + __shfl_xor(acc, 1);    // horizontal add: adjacent pairs
    acc = acc + __shfl_xor(acc, 2);    // horizontal add: the two pair sums

    if (valid && c == 0) {
        float v = acc;
        if (k & 31) v = add_tail(v, wrow, a, nsteps * 32, k);
        const int64_t rows_m = t.row0[m + 1] - t.row0[m];
        t.out[m][col * rows_m + r] = v;
    }
}

}  // namespace

hipError_t launch_vec_dot(const RowTable &t, int64_t k, const uint16_t *a, int64_t ncols, bool vec8,
                          hipStream_t stream)
{
    const int64_t total = t.row0[t.count];
    const int per = vec8 ? kV8Rows : kV1Rows;
    const int64_t bx = (total + per - 1) / per;
    // grid.y is limited to 65535: launch column chunks, each with its own
    // activation and output offsets.
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    for (int64_t c0 = 0; c0 < ncols; c0 += 65535) {
        const int64_t nc = ncols - c0 < 65535 ? ncols - c0 : 65535;
        RowTable tc = t;
        for (int i = 0; i < t.count; i++) tc.out[i] = t.out[i] + c0 * (t.row0[i + 1] - t.row0[i]);
        const dim3 grid((uint32_t)bx, (uint32_t)nc);
        if (vec8)
            vec_dot_v8<<<grid, dim3(256), 0, stream>>>(tc, k, a + c0 * k);
        else
            vec_dot_v1<<<grid, dim3(256), 0, stream>>>(tc, k, a + c0 * k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace f16wm
