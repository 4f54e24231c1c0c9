// Exact f16 -> f32 widening: elementwise, and of selected weight rows.
//
// bankML f16 page, Technical usage: `widen` converts f16 values exactly
// (F16C where present) and `dequantize_row` widens one F16 weight row to f32
// (ggml's get_rows: the embedding lookup, on the tied token_embd matrix when
// the model has no output matrix, bankML page "bankML/forward.rs", Summary).
// v_cvt_f32_f16 is exact for every finite f16, subnormals included (HIP keeps
// f16 denormals); NaNs stay NaNs.
//
// HBM-bound: 2 bytes read and 4 written per element.  One thread widens 8
// elements: one 16-byte load, two 16-byte stores.
#include "kernels.h"

namespace f16wm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void widen8(const uint16_t *src, float *dst)
{
    const half8 h = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4 *>(src));
    float4 lo, hi;
    lo.x = (float)h[0];
    lo.y = (float)h[1];
    lo.z = (float)h[2];
    lo.w = (float)h[3];
    hi.x = (float)h[4];
    hi.y = (float)h[5];
    hi.z = (float)h[6];
    hi.w = (float)h[7];
    *reinterpret_cast<float4 *>(dst) = lo;
    *reinterpret_cast<float4 *>(dst + 4) = hi;
}

template <bool kVec>
__global__ __launch_bounds__(256) void widen_kernel(const uint16_t *__restrict__ h, float *__restrict__ y,
                                                    int64_t count)
{
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= count) return;
    if (kVec && i0 + 8 <= count) {
        widen8(h + i0, y + i0);
        return;
    }
    const int64_t i1 = i0 + 8 < count ? i0 + 8 : count;
    for (int64_t i = i0; i < i1; i++) y[i] = (float)__builtin_bit_cast(_Float16, h[i]);
}

// Row ids[r] of W (rows x k) widened into out[r*k .. r*k + k).  An id outside
// [0, rows) fills its output row with quiet NaN.  grid: (ceil(k/8/256), nids).
template <bool kVec>
__global__ __launch_bounds__(256) void get_rows_kernel(const uint16_t *__restrict__ w, int64_t rows,
                                                       int64_t k, const int64_t *__restrict__ ids,
                                                       float *__restrict__ out)
{
    const int64_t r = blockIdx.y;
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= k) return;
    const int64_t id = ids[r];
    float *dst = out + r * k;
    const int64_t i1 = i0 + 8 < k ? i0 + 8 : k;
    if (id < 0 || id >= rows) {
        for (int64_t i = i0; i < i1; i++) dst[i] = __builtin_nanf("");
        return;
    }
    const uint16_t *src = w + id * k;
    if (kVec && i0 + 8 <= k) {
        widen8(src + i0, dst + i0);
        return;
    }
    for (int64_t i = i0; i < i1; i++) dst[i] = (float)__builtin_bit_cast(_Float16, src[i]);
}

}  // namespace

hipError_t launch_widen(const uint16_t *h, float *y, int64_t count, hipStream_t stream)
{
    const bool vec = ((uintptr_t)h % 16 == 0) && ((uintptr_t)y % 16 == 0);
    const int64_t blocks = ((count + 7) / 8 + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    if (vec)
        widen_kernel<true><<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(h, y, count);
    else
        widen_kernel<false><<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(h, y, count);
    return hipGetLastError();
}

hipError_t launch_get_rows(const uint16_t *w, int64_t rows, int64_t k, const int64_t *ids, int64_t nids,
                           float *out, hipStream_t stream)
{
    // 16-byte vectors need 16-byte aligned rows on both sides
    const bool vec = k % 8 == 0 && ((uintptr_t)w % 16 == 0) && ((uintptr_t)out % 16 == 0);
    const int64_t bx = ((k + 7) / 8 + 255) / 256;
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;
    for (int64_t r0 = 0; r0 < nids; r0 += 65535) {
        const int64_t nr = nids - r0 < 65535 ? nids - r0 : 65535;
        const dim3 grid((uint32_t)bx, (uint32_t)nr);
        if (vec)
            get_rows_kernel<true><<<grid, dim3(256), 0, stream>>>(w, rows, k, ids + r0, out + r0 * k);
        else
            get_rows_kernel<false><<<grid, dim3(256), 0, stream>>>(w, rows, k, ids + r0, out + r0 * k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace f16wm
