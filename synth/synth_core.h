/*
 * synth_core.h -- the seeded, counter-based input generator.
 *
 * Test and benchmark input infrastructure.  It holds none of the method's
 * arithmetic: only an integer hash, an integer approximation of a normal
 * draw, and an exact encoding of "integer x times 2^e" as a 16-bit pattern
 * (no rounding ever happens: the host checks that every value it asks for is
 * representable).  The same definitions compile for the host (gcc) and for
 * the device (hipcc), so both sides produce identical bits for any index.
 *
 * Hash: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), applied to
 * key + index * golden-gamma, i.e. SplitMix64's own state sequence.
 *
 * Normal draw: Irwin-Hall with four 16-bit uniforms taken from one hash,
 * centred; its standard deviation is sqrt(4 * (65536^2 - 1) / 12) ~ 37837.23
 * units, its tails are cut at about 3.46 sigma.  The centred sum d is scaled
 * by an integer multiplier M and shifted right by 16, keeping the sign, which
 * gives an integer x that the encoder turns into x * 2^e exactly.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN static inline __host__ __device__
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

/* Key of one stream: (seed, kind, step, rank) -> 64 bits. */
SYNTH_FN uint64_t synth_stream_key(uint64_t seed, uint64_t kind, uint64_t step, uint64_t rank) {
    uint64_t k = synth_mix64(seed ^ 0x5EEDC0DE5EEDC0DEULL);
    k = synth_mix64(k + kind * SYNTH_GOLDEN);
    k = synth_mix64(k + step * SYNTH_GOLDEN);
    k = synth_mix64(k + rank * SYNTH_GOLDEN);
    return k;
}

SYNTH_FN uint64_t synth_hash(uint64_t key, uint64_t index) {
    return synth_mix64(key + (index + 1) * SYNTH_GOLDEN);
}

/* Integer draw, roughly normal with sd 37837.23 * M / 65536, symmetric. */
SYNTH_FN int64_t synth_draw(uint64_t h, int64_t mult) {
    int64_t s = (int64_t)(h & 0xFFFF) + (int64_t)((h >> 16) & 0xFFFF) +
                (int64_t)((h >> 32) & 0xFFFF) + (int64_t)(h >> 48);
    int64_t d = s - 131070;
    int64_t a = d < 0 ? -d : d;
    int64_t x = (a * mult) >> 16;
    return d < 0 ? -x : x;
}

/* Exact 16-bit pattern of x * 2^e.  The caller guarantees |x| < 2^(frac_bits+1),
 * that x * 2^e is below the format's overflow threshold, and that 2^e is a
 * multiple of the smallest subnormal, so nothing is rounded. */
SYNTH_FN uint16_t synth_encode(int64_t x, int e, int exp_bits, int frac_bits) {
    if (x == 0) return 0;
    uint16_t sign = x < 0 ? 0x8000 : 0;
    uint64_t a = (uint64_t)(x < 0 ? -x : x);
    int bias = (1 << (exp_bits - 1)) - 1;
    int b = 63 - __builtin_clzll(a);          /* a = 1.f * 2^b            */
    int field = b + e + bias;
    if (field >= 1) {
        uint64_t mant = (a << (frac_bits - b)) & ((1ULL << frac_bits) - 1);
        return (uint16_t)(sign | ((uint64_t)field << frac_bits) | mant);
    }
    int shift = e - 1 + bias + frac_bits;     /* subnormal: a * 2^shift   */
    return (uint16_t)(sign | (a << shift));
}

/* One generated element at global flat index `index`. */
SYNTH_FN uint16_t synth_value(uint64_t key, uint64_t index, int64_t mult, int e,
                              int exp_bits, int frac_bits) {
    return synth_encode(synth_draw(synth_hash(key, index), mult), e, exp_bits, frac_bits);
}

#endif /* SYNTH_CORE_H */
