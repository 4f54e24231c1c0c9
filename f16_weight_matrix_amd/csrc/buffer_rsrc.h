// Buffer resources for raw buffer loads (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace f16wm {

// Raw buffer resource over `bytes` (< 2^31) from `base`: stride 0,
// num_records = bytes, so a load at an offset past the end reads zero.
// Both arguments are wave-uniform; readfirstlane lets the compiler keep the
// descriptor in SGPRs.  The halves go through uint32_t: readfirstlane
// returns int, and widening that straight to 64 bits would sign-extend the
// low word into the high one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int64_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const int nb = __builtin_amdgcn_readfirstlane((int)bytes);
    // dword3 = 0x00020000: the gfx9 data format for raw 32-bit access
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, nb, 0x00020000);
}

}  // namespace f16wm
