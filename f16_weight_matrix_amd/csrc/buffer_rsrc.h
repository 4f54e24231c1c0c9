// Buffer resources for raw buffer loads (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "addr_words.h"

namespace f16wm {

// Raw buffer resource over `bytes` (< 2^31) from `base`: stride 0,
// num_records = bytes, so a load at an offset past the end reads zero.
// Both arguments are wave-uniform; readfirstlane lets the compiler keep the
// descriptor in SGPRs.  The two address words are joined by join_words,
// which keeps the low word from being sign-extended into the high one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int64_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const int lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const int hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const int nb = __builtin_amdgcn_readfirstlane((int)bytes);
    // dword3 = 0x00020000: the gfx9 data format for raw 32-bit access
    return __builtin_amdgcn_make_buffer_rsrc((void *)join_words(lo, hi), (short)0, nb, 0x00020000);
}

}  // namespace f16wm
