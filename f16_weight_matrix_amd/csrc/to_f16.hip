// Activation rounding: binary32 -> binary16, round to nearest even
// (bankML f16 page, Design notes, "Activation"; the rounding itself is
// rne_f16 in f16_round.h, shared with the fused-activation products).
//
// HBM-bound: 4 bytes in, 2 bytes out per element.  Each thread converts eight
// elements with two 16-byte loads and one 16-byte store.
#include "f16_round.h"
#include "kernels.h"

namespace f16wm {
namespace {

template <bool kVec>
__global__ __launch_bounds__(256) void to_f16_kernel(const float *__restrict__ x,
                                                     uint16_t *__restrict__ y, int64_t count)
{
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= count) return;
    if (kVec && i0 + 8 <= count) {
        const float4 p = *reinterpret_cast<const float4 *>(x + i0);
        const float4 q = *reinterpret_cast<const float4 *>(x + i0 + 4);
        uint4 o;
        o.x = (uint32_t)rne_f16(p.x) | ((uint32_t)rne_f16(p.y) << 16);
        o.y = (uint32_t)rne_f16(p.z) | ((uint32_t)rne_f16(p.w) << 16);
        o.z = (uint32_t)rne_f16(q.x) | ((uint32_t)rne_f16(q.y) << 16);
        o.w = (uint32_t)rne_f16(q.z) | ((uint32_t)rne_f16(q.w) << 16);
        *reinterpret_cast<uint4 *>(y + i0) = o;
        return;
    }
    const int64_t i1 = i0 + 8 < count ? i0 + 8 : count;
    for (int64_t i = i0; i < i1; i++) y[i] = rne_f16(x[i]);
}

}  // namespace

hipError_t launch_to_f16(const float *x, uint16_t *y, int64_t count, hipStream_t stream)
{
    const bool vec = ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0);
    const int64_t threads = (count + 7) / 8;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;   // grid.x limit
    if (vec)
        to_f16_kernel<true><<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(x, y, count);
    else
        to_f16_kernel<false><<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(x, y, count);
    return hipGetLastError();
}

}  // namespace f16wm
