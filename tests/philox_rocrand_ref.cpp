// Prints Philox4x32-10 blocks computed by rocRAND's header engine, for counters read
// from stdin as "c0 c1 c2 c3 k0 k1" lines.  An independent implementation used only
// to pin the CPU oracle's Philox; it is never part of the library.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        const unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
        const unsigned long long subsequence = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
        const unsigned long long block = (unsigned long long)c0 | ((unsigned long long)c1 << 32);
        // The engine's counter is (offset/4 in words 0-1, subsequence in words 2-3).
        rocrand_device::philox4x32_10_engine eng(seed, subsequence, 4ull * block);
        unsigned x0 = eng(), x1 = eng(), x2 = eng(), x3 = eng();
        std::printf("%u %u %u %u\n", x0, x1, x2, x3);
    }
    return 0;
}
