// The activation rounding shared by every kernel that rounds f32 to f16.
//
// bankML f16 page, Design notes ("Activation"): round to nearest, ties to
// even (F16C vcvtps2ph with immediate 0).  v_cvt_f16_f32 rounds by the MODE
// register (round-to-nearest-even in HIP kernels), keeps f16 subnormals and
// overflows to infinity; NaN is re-encoded explicitly as a quiet NaN keeping
// the sign and the top ten payload bits, as F16C does.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace f16wm {

__device__ __forceinline__ uint16_t rne_f16(float x)
{
    uint32_t b = __float_as_uint(x);
    uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)x);
    if ((b & 0x7fffffffu) > 0x7f800000u)
        h = (uint16_t)(((b >> 16) & 0x8000u) | 0x7e00u | ((b >> 13) & 0x3ffu));
    return h;
}

// The same rounding of an f32 value the kernel has just computed (a product
// or an FMA).  The empty asm makes the value opaque, so the compiler cannot
// fuse the operation that produced it with the conversion: it would emit
// v_fma_mixlo_f16 / v_mad_mixlo_f16, one rounding from the exact result
// straight to f16, which differs from rounding to f32 first at f16 ties.
__device__ __forceinline__ uint16_t rne_f16_of_result(float x)
{
    asm("" : "+v"(x));
    return rne_f16(x);
}

}  // namespace f16wm
