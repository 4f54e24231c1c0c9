// A 64-bit address from two 32-bit words (host and device; no HIP header, so
// a host test can include it with the attribute macros defined empty).
#pragma once
#include <stdint.h>

namespace f16wm {

// The value whose low word is `lo` and high word is `hi`, each taken as an
// unsigned 32-bit word.  The words come from __builtin_amdgcn_readfirstlane,
// which returns int: widening an int straight to 64 bits copies bit 31 of the
// low word into the whole high word, a wrong address whenever that bit is
// set (a buffer anywhere in the upper half of a 4 GiB window).
__host__ __device__ __forceinline__ uint64_t join_words(int lo, int hi)
{
    return ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

}  // namespace f16wm
