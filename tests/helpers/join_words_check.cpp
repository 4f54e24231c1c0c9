// Host check of f16wm::join_words (csrc/addr_words.h): the 64-bit address a
// buffer resource is built from, joined from the two int words that
// readfirstlane returns.  Prints one line per case and exits non-zero on the
// first wrong join.
#define __host__
#define __device__
#define __forceinline__ inline
#include <stdio.h>

#include "addr_words.h"

int main()
{
    // (address, low word with bit 31 set or not)
    const uint64_t cases[] = {
        0x00007f1234567890ull, 0x00007f12b4567890ull, 0x0000000080000000ull, 0x00000001ffffffffull,
        0x00007fff80000000ull, 0x0000000000000000ull, 0x00007fffffffffffull, 0x0000555500000001ull,
    };
    int bad = 0;
    for (uint64_t p : cases) {
        const int lo = (int)(uint32_t)p;              // what readfirstlane hands back
        const int hi = (int)(uint32_t)(p >> 32);
        const uint64_t got = f16wm::join_words(lo, hi);
        printf("%016llx -> %016llx%s\n", (unsigned long long)p, (unsigned long long)got, got == p ? "" : "  WRONG");
        bad += got != p;
    }
    return bad ? 1 : 0;
}
