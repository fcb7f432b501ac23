/* Host sanitizer run of the oracle (test infrastructure): every oracle
 * function on random shapes, each buffer allocated at exactly its size so
 * that AddressSanitizer reports any access outside it and UBSan any
 * undefined arithmetic.  Built and run by tests/test_oracle_sanitizers.py
 * with gcc -fsanitize=address,undefined; prints "ok" on success. */
#include "../oracle/oracle.c"

#include <stdio.h>
#include <stdlib.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {            /* SplitMix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t below(int64_t n) { return n > 0 ? (int64_t)(next_u64() % (uint64_t)n) : 0; }

static uint16_t* rand16(int64_t n) {
    uint16_t* a = (uint16_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint16_t));
    for (int64_t i = 0; i < n; ++i) a[i] = (uint16_t)next_u64();
    return a;
}

int main(void) {
    for (int iter = 0; iter < 300; ++iter) {
        /* layout and buckets */
        const int64_t nt = below(12);
        int64_t* numel = (int64_t*)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int64_t));
        for (int64_t k = 0; k < nt; ++k) numel[k] = below(3000);
        const int32_t world = 1 + (int32_t)below(16);
        const int32_t align = 1 + (int32_t)below(8);
        int64_t* off = (int64_t*)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int64_t));
        int64_t* parts = (int64_t*)malloc((size_t)(world + 1) * sizeof(int64_t));
        int64_t padded = 0;
        if (oracle_layout(numel, nt, world, align, off, parts, &padded) != O_OK) return 1;
        int64_t* first = (int64_t*)malloc((size_t)(nt + 1) * sizeof(int64_t));
        int64_t nb = 0;
        if (oracle_buckets(numel, nt, 1 + below(5000), first, &nb) != O_OK) return 2;
        /* copy-in / write-back over the layout */
        uint16_t** tens = (uint16_t**)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(uint16_t*));
        for (int64_t k = 0; k < nt; ++k) tens[k] = rand16(numel[k]);
        uint16_t* flat = rand16(padded);
        oracle_flat_gather(flat, padded, (const uint16_t* const*)tens, off, numel, nt);
        oracle_flat_scatter(flat, tens, off, numel, nt);
        /* reduce, check, AdamW on one partition */
        const int64_t count = parts[1] - parts[0];
        const int32_t dtype = 1 + (int32_t)(iter & 1);
        const int32_t nr = 1 + (int32_t)below(16);
        uint16_t* src[16];
        for (int r = 0; r < nr; ++r) src[r] = rand16(count);
        uint16_t* red = rand16(count);
        oracle_reduce(red, (const uint16_t* const*)src, nr, count, dtype);
        uint32_t ovf = 0;
        double sumsq = 0.0;
        oracle_check(red, count, dtype, 1.0f / 1024.0f, &ovf, &sumsq);
        float* master = (float*)malloc((size_t)(count > 0 ? count : 1) * sizeof(float));
        float* m = (float*)calloc((size_t)(count > 0 ? count : 1), sizeof(float));
        float* v = (float*)calloc((size_t)(count > 0 ? count : 1), sizeof(float));
        uint16_t* p16 = rand16(count);
        oracle_init_master(master, p16, count, dtype);
        oracle_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1.0f, 1 + below(100)};
        oracle_adamw(master, m, v, p16, red, count, dtype, 1.0f / 1024.0f, sumsq, 0, &hp);
        double* mo = (double*)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
        double* mm = (double*)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
        double* vv = (double*)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
        oracle_adamw_f64(master, m, v, red, count, dtype, 1.0 / 1024.0, 1.0, &hp, mo, mm, vv);
        /* converters */
        double* dec = (double*)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
        oracle_decode16(red, dec, count, dtype);
        oracle_encode16_from_f64(dec, p16, count, dtype);
        oracle_encode16_from_f32(master, p16, count, dtype);
        oracle_scaler sc = {65536.0, 1.0, 3, 0, 0};
        for (int k = 0; k < 20; ++k) oracle_scaler_update(&sc, (uint32_t)(next_u64() & 1));
        (void)oracle_clip_coef(1.0f, sumsq);
        free(dec); free(vv); free(mm); free(mo); free(p16); free(v); free(m); free(master);
        free(red);
        for (int r = 0; r < nr; ++r) free(src[r]);
        free(flat);
        for (int64_t k = 0; k < nt; ++k) free(tens[k]);
        free(tens); free(first); free(parts); free(off); free(numel);
    }
    printf("ok\n");
    return 0;
}
