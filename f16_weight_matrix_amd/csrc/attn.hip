// The f16 attention helpers over an f16 KV cache: vec_dot_u16 scores against
// the K cache, and the V-accumulator updates mad and scale.
//
// bankML f16 page, Summary and Technical usage: the attention code uses
// vec_dot_u16 (the vec_dot order with the first operand given as f16 values)
// for K-cache rows, and mad (ggml_vec_mad_f16) and scale (ggml_vec_scale_f16)
// for the f16 V accumulator.
//
// kq: out[h][p] = vec_dot(K[p][h / G], q[h]) with the cache laid out
// position-major, K[p][j][0..d), and G = n_head / n_kv_head query heads per
// KV head.  A block takes one KV head and a run of positions; its 256 threads
// form pairs (position, query head) of LPR lanes, lane j of a pair owning
// chains CPL*j .. CPL*j + CPL - 1 (CPL = 32 / LPR) of that element.  With
// d % 8 == 0 and 16-byte rows (LPR = 4) a lane reads, per 32-element step,
// the 16 bytes of its chains from the K row and from the query; the G pairs of
// one position read the same K bytes, which the same or neighbouring wave
// loads serve from L1.  Pairs are laid out query-major, so each wave's stores
// are consecutive positions of one score row.  The reduction is the vec_dot
// tree (vec_dot_order.h); the d % 32 tail is added in binary64 by lane 0.
// HBM-bound: the cache is read once, 2 * n_kv * n_kv_head * d bytes.
//
// mad / scale: element-wise over nvec vectors of n f16 values with one f32
// weight (factor) per vector: acc = f16(fma(f32(v), w, f32(acc))) and
// acc = f16(f32(acc) * s), the f16 rounding being the activation rounding
// (f16_round.h) applied to the finished f32 result (rne_f16_of_result keeps
// the compiler from fusing the two roundings into one mixed-precision
// instruction).  HBM-bound: 6 (mad) or 4 (scale) bytes per element.
#include "f16_round.h"
#include "kernels.h"
#include "vec_dot_order.h"

namespace f16wm {
namespace {

template <int LPR>
__global__ __launch_bounds__(256) void kq_kernel(const uint16_t *__restrict__ kc, int64_t n_kv, int64_t n_kv_head,
                                                 int64_t d, const uint16_t *__restrict__ q, int64_t G, int P,
                                                 int GB, float *__restrict__ out)
{
    constexpr int CPL = 32 / LPR;
    typedef typename Halves<CPL>::T HT;
    const int tid = threadIdx.x;
    const int pair = tid / LPR;
    const int jj = tid % LPR;
    const int gl = pair / P;                       // query head within this block
    const int pp = pair % P;                       // position within this block
    const int64_t j = blockIdx.y;                  // KV head
    const int64_t g = (int64_t)blockIdx.z * GB + gl;
    const int64_t p = (int64_t)blockIdx.x * P + pp;
    const bool valid = gl < GB && g < G && p < n_kv;
    const int64_t h = j * G + (valid ? g : 0);
    const uint16_t *krow = kc + ((valid ? p : 0) * n_kv_head + j) * d;
    const uint16_t *qrow = q + h * d;

    const int64_t nsteps = d >> 5;
    float acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; i++) acc[i] = 0.f;
    if (valid) {
        for (int64_t t = 0; t < nsteps; t++) {
            const int64_t e = 32 * t + CPL * jj;
            fma_halves<CPL>(acc, *reinterpret_cast<const HT *>(krow + e), *reinterpret_cast<const HT *>(qrow + e));
        }
    }
    float v = vec_dot_tree<CPL>(acc);              // every lane of the pair takes part
    if (valid && jj == 0) {
        if (d & 31) {
            double s = (double)v;
            for (int64_t i = nsteps * 32; i < d; i++) s = s + (double)(widen(krow[i]) * widen(qrow[i]));
            v = (float)s;
        }
        out[h * n_kv + p] = v;
    }
}

// Eight elements per thread (n % 8 == 0, 16-byte aligned arrays) or one.
template <bool kVec8>
__global__ __launch_bounds__(256) void mad_kernel(uint16_t *__restrict__ acc, const uint16_t *__restrict__ v,
                                                  const float *__restrict__ w, int64_t nvec, int64_t n)
{
    const int64_t total = nvec * n;
    const int64_t per = kVec8 ? 8 : 1;
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * per; e < total;
         e += (int64_t)gridDim.x * 256 * per) {
        const float wb = w[e / n];
        if (kVec8) {
            const half8 a = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4 *>(acc + e));
            const half8 x = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4 *>(v + e));
            uint16_t r[8];
#pragma unroll
            for (int i = 0; i < 8; i++) r[i] = rne_f16_of_result(__builtin_fmaf((float)x[i], wb, (float)a[i]));
            u32x4 o;
            o[0] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
            o[1] = (uint32_t)r[2] | ((uint32_t)r[3] << 16);
            o[2] = (uint32_t)r[4] | ((uint32_t)r[5] << 16);
            o[3] = (uint32_t)r[6] | ((uint32_t)r[7] << 16);
            *reinterpret_cast<u32x4 *>(acc + e) = o;
        } else {
            acc[e] = rne_f16_of_result(__builtin_fmaf(widen(v[e]), wb, widen(acc[e])));
        }
    }
}

template <bool kVec8>
__global__ __launch_bounds__(256) void scale_kernel(uint16_t *__restrict__ acc, const float *__restrict__ s,
                                                    int64_t nvec, int64_t n)
{
    const int64_t total = nvec * n;
    const int64_t per = kVec8 ? 8 : 1;
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * per; e < total;
         e += (int64_t)gridDim.x * 256 * per) {
        const float sb = s[e / n];
        if (kVec8) {
            const half8 a = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4 *>(acc + e));
            uint16_t r[8];
#pragma unroll
            for (int i = 0; i < 8; i++) r[i] = rne_f16_of_result((float)a[i] * sb);
            u32x4 o;
            o[0] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
            o[1] = (uint32_t)r[2] | ((uint32_t)r[3] << 16);
            o[2] = (uint32_t)r[4] | ((uint32_t)r[5] << 16);
            o[3] = (uint32_t)r[6] | ((uint32_t)r[7] << 16);
            *reinterpret_cast<u32x4 *>(acc + e) = o;
        } else {
            acc[e] = rne_f16_of_result(widen(acc[e]) * sb);
        }
    }
}

// Enough blocks to fill the GPU several times over; the kernels stride.
uint32_t elementwise_grid(int64_t items)
{
    const int64_t blocks = (items + 255) / 256;
    return (uint32_t)(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192);
}

}  // namespace

hipError_t launch_kq(const uint16_t *kc, int64_t n_kv, int64_t n_kv_head, int64_t d, const uint16_t *q,
                     int64_t n_head, bool vec8, float *out, hipStream_t stream)
{
    const int lpr = vec8 ? 4 : 32;
    const int pairs = 256 / lpr;                   // pairs per block
    const int64_t G = n_head / n_kv_head;
    const int GB = (int)(G < pairs ? G : pairs);   // query heads per block
    const int P = pairs / GB;                      // positions per block
    const int64_t gx = (n_kv + P - 1) / P, gz = (G + GB - 1) / GB;
    if (gx > 0x7fffffff || n_kv_head > 65535 || gz > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)gx, (uint32_t)n_kv_head, (uint32_t)gz);
    if (vec8)
        kq_kernel<4><<<grid, dim3(256), 0, stream>>>(kc, n_kv, n_kv_head, d, q, G, P, GB, out);
    else
        kq_kernel<32><<<grid, dim3(256), 0, stream>>>(kc, n_kv, n_kv_head, d, q, G, P, GB, out);
    return hipGetLastError();
}

hipError_t launch_mad(uint16_t *acc, const uint16_t *v, const float *w, int64_t nvec, int64_t n, bool vec8,
                      hipStream_t stream)
{
    const int64_t items = vec8 ? nvec * n / 8 : nvec * n;
    const dim3 grid(elementwise_grid(items));
    if (vec8)
        mad_kernel<true><<<grid, dim3(256), 0, stream>>>(acc, v, w, nvec, n);
    else
        mad_kernel<false><<<grid, dim3(256), 0, stream>>>(acc, v, w, nvec, n);
    return hipGetLastError();
}

hipError_t launch_scale(uint16_t *acc, const float *s, int64_t nvec, int64_t n, bool vec8, hipStream_t stream)
{
    const int64_t items = vec8 ? nvec * n / 8 : nvec * n;
    const dim3 grid(elementwise_grid(items));
    if (vec8)
        scale_kernel<true><<<grid, dim3(256), 0, stream>>>(acc, s, nvec, n);
    else
        scale_kernel<false><<<grid, dim3(256), 0, stream>>>(acc, s, nvec, n);
    return hipGetLastError();
}

}  // namespace f16wm
