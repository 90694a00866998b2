// Reference Philox4x32-10 outputs from rocRAND's host-callable engine, used by
// the oracle pins as a library routine. Reads lines "k0 k1 c0 c1 c2 c3" (hex)
// from stdin and prints the four output words of that (key, counter).
//
// rocRAND's engine keys itself with the 64-bit seed (low word first), starts its
// counter at zero, adds the subsequence to counter words 2..3 and offset / 4 to
// words 0..1; so seed = k0 | k1 << 32, subsequence = c2 | c3 << 32 and
// offset = 4 (c0 | c1 << 32) place the engine exactly at (key, counter).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
    unsigned k0, k1, c0, c1, c2, c3;
    while (std::scanf("%x %x %x %x %x %x", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        const unsigned long long seed = k0 | (static_cast<unsigned long long>(k1) << 32);
        const unsigned long long sub = c2 | (static_cast<unsigned long long>(c3) << 32);
        const unsigned long long ctr = c0 | (static_cast<unsigned long long>(c1) << 32);
        rocrand_device::philox4x32_10_engine eng(seed, sub, 0);
        eng.discard(ctr * 4);  // offset in numbers: four per counter value
        const unsigned a = eng.next(), b = eng.next(), c = eng.next(), d = eng.next();
        std::printf("%08x %08x %08x %08x\n", a, b, c, d);
    }
    return 0;
}
