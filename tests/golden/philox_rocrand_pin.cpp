// Independent Philox4x32-10 for pinning the oracle: rocRAND's host-callable
// engine. Reads lines "key0 key1 c0 c1 c2 c3" (hex) on stdin and prints the four
// output words of Philox4x32-10(counter = (c0, c1, c2, c3), key = (key0, key1)).
// rocRAND's engine keys on the 64-bit seed (low word = key0) and, for
// subsequence s and offset o, starts at counter (o/4 low, o/4 high, s low, s high).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned k0, k1, c0, c1, c2, c3;
    while (std::scanf("%x %x %x %x %x %x", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
        unsigned long long subseq = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
        unsigned long long offset = 4ull * ((unsigned long long)c0 | ((unsigned long long)c1 << 32));
        rocrand_device::philox4x32_10_engine e(seed, subseq, offset);
        unsigned w0 = e.next(), w1 = e.next(), w2 = e.next(), w3 = e.next();
        std::printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
    }
    return 0;
}
