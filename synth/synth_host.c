/*
 * synth_host.c -- host side of the seeded input generator (see synth_core.h).
 * Built with gcc into libsynth_host.so; the Python wrapper releases the GIL
 * around these calls, so disjoint index ranges can be filled from threads.
 */
#include "synth_core.h"

uint64_t synth_key(uint64_t seed, uint64_t kind, uint64_t step, uint64_t rank) {
    return synth_stream_key(seed, kind, step, rank);
}

uint64_t synth_hash64(uint64_t key, uint64_t index) { return synth_hash(key, index); }

/* out[j] = value at global index first + j, j in [0, n). */
void synth_fill(uint16_t* out, int64_t n, uint64_t first, uint64_t key, int64_t mult, int32_t e,
                int32_t exp_bits, int32_t frac_bits) {
    for (int64_t j = 0; j < n; ++j)
        out[j] = synth_value(key, first + (uint64_t)j, mult, e, exp_bits, frac_bits);
}

/* out[j] = value at global index idx[j] (gathered samples). */
void synth_gather(uint16_t* out, const int64_t* idx, int64_t n, uint64_t key, int64_t mult,
                  int32_t e, int32_t exp_bits, int32_t frac_bits) {
    for (int64_t j = 0; j < n; ++j)
        out[j] = synth_value(key, (uint64_t)idx[j], mult, e, exp_bits, frac_bits);
}
