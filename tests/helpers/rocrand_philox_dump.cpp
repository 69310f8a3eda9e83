// Prints raw Philox4x32-10 words from rocRAND's header-only engine, run on
// the host.  Used only by the oracle's Philox pin: an implementation written
// by someone else, compared word for word.
//   usage: rocrand_philox_dump <seed> <subsequence> <offset> <calls>
// Each line holds the four words of one rocrand4() call.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
    if (argc != 5) return 2;
    unsigned long long seed = strtoull(argv[1], nullptr, 0);
    unsigned long long sub = strtoull(argv[2], nullptr, 0);
    unsigned long long off = strtoull(argv[3], nullptr, 0);
    long calls = strtol(argv[4], nullptr, 0);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, off, &st);
    for (long i = 0; i < calls; ++i) {
        uint4 v = rocrand4(&st);
        printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
    }
    return 0;
}
