/*
 * oracle.c -- plain scalar CPU oracle for the ZeRO-1/2 owner-shard step.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only tests/, __graft_entry__.smoke()
 * and bench.py's cpu_baseline leg may load it.  It shares no code, header or
 * table with the HIP library; neither includes the other.
 *
 * Every routine is the definition written out, one element at a time, in the
 * order the pages give the method:
 *
 *   layout   flatten a parameter group, pad it to the alignment, cut it into
 *            N equal partitions          (ZeRO-2 source walkthrough, discosf.com,
 *                                          sections 2.1 and 4.1)
 *   reduce   the owner receives the sum of every rank's gradient for its slice
 *                                        (ZeRO 优化器, cookllm.com, "ZeRO Stage 1",
 *                                          gradient-state list after reduce)
 *   check    overflow test + squared L2 norm of the unscaled gradient
 *                                        (wmrh.cn ZeRO article, section 3.1 fp16
 *                                          block and section 3.3 gradient_clipping)
 *   adamw    decoupled-weight-decay Adam on the fp32 master partition, then the
 *            16-bit copy                 (ZeRO-2 source walkthrough, sections 4.1
 *                                          and 4.3; hyper-parameters from the
 *                                          wmrh.cn article section 3.1 ds_config)
 *
 * Precision.  The pages fix the storage types: 16-bit parameters and gradients,
 * fp32 master weights, m and v (ZeRO / DeepSpeed 深度解读报告 section 2.1 table;
 * ZeRO 优化器 "训练状态的冗余分析").  The optimizer runs on the fp32 partition, so
 * its per-element arithmetic is fp32, one IEEE rounding per operation, no fused
 * multiply-add (build with -ffp-contract=off).  Everything the pages leave open
 * is read as follows: the gradient sum is taken in fp32, in rank order from +0,
 * and rounded once to 16 bits; the unscaled gradient is the fp32 product of the
 * value and 1/(S*D); the norm and the scalar constants are computed in fp64,
 * each rounded once to its storage type.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define O_OK 0
#define O_EINVAL (-1)
#define O_ERANGE (-2)

#define O_FP16 1
#define O_BF16 2

/* ------------------------------------------------------------------------- */
/* 16-bit formats, from their definitions.                                   */
/*   binary16 (IEEE 754): 1 sign bit, 5 exponent bits (bias 15), 10 fraction */
/*   bfloat16:            1 sign bit, 8 exponent bits (bias 127), 7 fraction */
/* ------------------------------------------------------------------------- */
typedef struct {
    int exp_bits;
    int frac_bits;
} fmt16;

static fmt16 fmt_of(int32_t dtype) {
    fmt16 f;
    if (dtype == O_BF16) { f.exp_bits = 8; f.frac_bits = 7; }
    else { f.exp_bits = 5; f.frac_bits = 10; }
    return f;
}

/* The exact value of a 16-bit pattern. */
static double decode16(uint16_t h, fmt16 f) {
    int bias = (1 << (f.exp_bits - 1)) - 1;
    int emax = (1 << f.exp_bits) - 1;
    int sign = h >> 15;
    int e = (h >> f.frac_bits) & emax;
    int frac = h & ((1 << f.frac_bits) - 1);
    double v;
    if (e == emax)
        v = frac ? NAN : INFINITY;
    else if (e == 0)                      /* subnormal: frac * 2^(1-bias-fb) */
        v = ldexp((double)frac, 1 - bias - f.frac_bits);
    else                                  /* normal: 1.frac * 2^(e-bias)      */
        v = ldexp((double)((1 << f.frac_bits) + frac), e - bias - f.frac_bits);
    return sign ? -v : v;
}

/* Round a real number (given as a double) to the nearest 16-bit value,
 * ties to even.  Overflow gives +-inf, subnormal results are kept, a NaN
 * becomes the quiet NaN with the input's sign. */
static uint16_t encode16(double x, fmt16 f) {
    int bias = (1 << (f.exp_bits - 1)) - 1;
    int emax = (1 << f.exp_bits) - 1;
    int fb = f.frac_bits;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | (emax << fb) | (1 << (fb - 1)));
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | (emax << fb));
    if (a == 0.0) return sign;

    int e2;
    frexp(a, &e2);                 /* a lies in [2^(e2-1), 2^e2)             */
    int E = e2 - 1;
    int emin = 1 - bias;           /* exponent of the smallest normal        */
    if (E < emin) E = emin;        /* subnormals share the smallest quantum  */
    int q = E - fb;                /* weight of the last kept bit is 2^q     */

    double scaled = ldexp(a, -q);  /* exact: only the exponent moves         */
    double r = floor(scaled);
    double rem = scaled - r;       /* exact fractional part                  */
    if (rem > 0.5 || (rem == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;

    if (r >= ldexp(1.0, fb + 1)) { /* rounding carried into the next binade  */
        r = r / 2.0;
        q += 1;
    }
    if (r < ldexp(1.0, fb))        /* still below the smallest normal        */
        return (uint16_t)(sign | (uint16_t)r);
    int field = q + fb + bias;     /* biased exponent of r * 2^q             */
    if (field >= emax) return (uint16_t)(sign | (emax << fb));
    return (uint16_t)(sign | (field << fb) | ((uint16_t)r - (1 << fb)));
}

/* decode16 of every pattern, built once from the definition above. */
static double g_value_table[3][65536];
static int g_table_ready[3];

static const double* value_table(int32_t dtype) {
    int k = (dtype == O_BF16) ? 2 : 1;
    if (!g_table_ready[k]) {
        fmt16 f = fmt_of(dtype);
        for (uint32_t h = 0; h < 65536u; ++h) g_value_table[k][h] = decode16((uint16_t)h, f);
        g_table_ready[k] = 1;
    }
    return g_value_table[k];
}

/* Exported converters so the tests can pin them against numpy / torch. */
void oracle_decode16(const uint16_t* in, double* out, int64_t n, int32_t dtype) {
    fmt16 f = fmt_of(dtype);
    for (int64_t i = 0; i < n; ++i) out[i] = decode16(in[i], f);
}

void oracle_encode16_from_f32(const float* in, uint16_t* out, int64_t n, int32_t dtype) {
    fmt16 f = fmt_of(dtype);
    for (int64_t i = 0; i < n; ++i) out[i] = encode16((double)in[i], f);
}

void oracle_encode16_from_f64(const double* in, uint16_t* out, int64_t n, int32_t dtype) {
    fmt16 f = fmt_of(dtype);
    for (int64_t i = 0; i < n; ++i) out[i] = encode16(in[i], f);
}

/* ------------------------------------------------------------------------- */
/* Layout: flatten, align, partition.                                        */
/* ZeRO-2 source walkthrough (discosf.com) section 4.1: the group's tensors   */
/* are concatenated into one flat buffer, aligned to a start-alignment factor */
/* (2 elements of 16-bit data), and split into as many partitions as there   */
/* are data-parallel ranks; section 2.1 calls them near-equal.  Reading: the  */
/* tail is padded to a multiple of N*A and every partition has P = padded/N   */
/* elements; tensors sit back to back with no padding between them.          */
/* ------------------------------------------------------------------------- */
int oracle_layout(const int64_t* numel, int64_t n_tensors, int32_t world, int32_t align,
                  int64_t* tensor_offset, int64_t* part_begin, int64_t* padded_total) {
    if (n_tensors < 0 || world < 1 || align < 1) return O_EINVAL;
    if (n_tensors > 0 && (numel == 0 || tensor_offset == 0)) return O_EINVAL;
    if (part_begin == 0 || padded_total == 0) return O_EINVAL;

    int64_t total = 0;
    for (int64_t k = 0; k < n_tensors; ++k) {
        if (numel[k] < 0) return O_EINVAL;
        tensor_offset[k] = total;
        if (total > INT64_MAX - numel[k]) return O_ERANGE;
        total += numel[k];
    }
    int64_t unit = (int64_t)world * (int64_t)align;
    int64_t groups = total / unit + (total % unit != 0);
    if (groups > INT64_MAX / unit) return O_ERANGE;
    int64_t padded = groups * unit;
    int64_t part = padded / world;
    for (int32_t p = 0; p <= world; ++p) part_begin[p] = (int64_t)p * part;
    *padded_total = padded;
    return O_OK;
}

/* Reduce buckets: tensors are taken in order into buckets of at most
 * `cap` elements; a bucket that cannot take the next whole tensor is closed
 * (ZeRO-2 source walkthrough section 4.2: gradients gather in a bucket of
 * reduce_bucket_size and the bucket is reduced when full).  A tensor larger
 * than the cap fills a bucket of its own.  bucket_first[b] is the first
 * tensor of bucket b; bucket_first[n_buckets] = n_tensors. */
int oracle_buckets(const int64_t* numel, int64_t n_tensors, int64_t cap,
                   int64_t* bucket_first, int64_t* n_buckets) {
    if (n_tensors < 0 || cap < 1 || bucket_first == 0 || n_buckets == 0) return O_EINVAL;
    int64_t nb = 0, fill = 0;
    for (int64_t k = 0; k < n_tensors; ++k) {
        if (numel[k] < 0) return O_EINVAL;
        if (k == 0 || (fill > 0 && fill + numel[k] > cap)) {
            bucket_first[nb++] = k;
            fill = 0;
        }
        fill += numel[k];
    }
    bucket_first[nb] = n_tensors;
    *n_buckets = nb;
    return O_OK;
}

/* ------------------------------------------------------------------------- */
/* Bucket copy-in and write-back.                                            */
/* ZeRO-2 source walkthrough (discosf.com) section 2.4: with                  */
/* contiguous_gradients the gradients are copied into one contiguous buffer;  */
/* section 4.2: each ready gradient goes into the reduce bucket at its place  */
/* in the flattened group; section 4.4: after the step the updated partitions */
/* are gathered back into the full parameters.                                */
/* gather:  flat[offset[k] + j] = tensor_k[j] for j < numel[k]; every flat    */
/*          element that no tensor covers becomes 0.                          */
/* scatter: tensor_k[j] = flat[offset[k] + j] for j < numel[k].               */
/* Elements are copied as 16-bit patterns, unchanged.                         */
/* ------------------------------------------------------------------------- */
void oracle_flat_gather(uint16_t* flat, int64_t flat_count, const uint16_t* const* tensors,
                        const int64_t* offset, const int64_t* numel, int64_t n_tensors) {
    for (int64_t i = 0; i < flat_count; ++i) flat[i] = 0;
    for (int64_t k = 0; k < n_tensors; ++k)
        for (int64_t j = 0; j < numel[k]; ++j) flat[offset[k] + j] = tensors[k][j];
}

void oracle_flat_scatter(const uint16_t* flat, uint16_t* const* tensors, const int64_t* offset,
                         const int64_t* numel, int64_t n_tensors) {
    for (int64_t k = 0; k < n_tensors; ++k)
        for (int64_t j = 0; j < numel[k]; ++j) tensors[k][j] = flat[offset[k] + j];
}

/* ------------------------------------------------------------------------- */
/* Reduce: red[i] = the sum over ranks r = 0..N-1 of g_r[i], rounded once to   */
/* the 16-bit communication type.  ZeRO 优化器, "ZeRO Stage 1": after the      */
/* reduce the owner holds the sum of every rank's gradient.  ZeRO-2 source     */
/* walkthrough section 三: with reduce-scatter the communicated type is        */
/* fp16/bf16.  The pages leave the accumulation open; it is read as fp32       */
/* additions in rank order starting from +0, each rounded to nearest-even,    */
/* then one rounding of the fp32 sum to the 16-bit type.  Every 16-bit value  */
/* is exactly a float, so each addend enters unchanged.                        */
/* ------------------------------------------------------------------------- */
void oracle_reduce(uint16_t* red, const uint16_t* const* src, int32_t n_ranks,
                   int64_t count, int32_t dtype) {
    const double* val = value_table(dtype);
    fmt16 f = fmt_of(dtype);
    for (int64_t i = 0; i < count; ++i) {
        float acc = 0.0f;
        for (int32_t r = 0; r < n_ranks; ++r) acc = acc + (float)val[src[r][i]];
        red[i] = encode16((double)acc, f);
    }
}

/* ------------------------------------------------------------------------- */
/* Check: overflow = some element of the reduced slice is inf or NaN;         */
/* sumsq = sum of g^2 in fp64, g = value * inv_scale as an fp32 product (each */
/* square is exact in fp64).                                                  */
/* wmrh.cn article section 3.1: fp16 training with dynamic loss scaling;      */
/* section 3.3: gradient_clipping.  Results are accumulated into *overflow    */
/* and *sumsq so several owner ranges can form one global result.             */
/* ------------------------------------------------------------------------- */
void oracle_check(const uint16_t* red, int64_t count, int32_t dtype, float inv_scale,
                  uint32_t* overflow, double* sumsq) {
    const double* val = value_table(dtype);
    uint32_t flag = *overflow;
    double s = *sumsq;
    for (int64_t i = 0; i < count; ++i) {
        double x = val[red[i]];
        if (!isfinite(x)) flag = 1;
        double g = (double)((float)x * inv_scale);
        s = s + g * g;
    }
    *overflow = flag;
    *sumsq = s;
}

/* Global-norm clip factor, as torch.nn.utils.clip_grad_norm_ documents it:
 * max_norm / (norm + 1e-6), applied only when below one.  Off when
 * max_norm <= 0. */
float oracle_clip_coef(float max_norm, double sumsq) {
    if (!(max_norm > 0.0f)) return 1.0f;
    double c = (double)max_norm / (sqrt(sumsq) + 1e-6);
    return c < 1.0 ? (float)c : 1.0f;
}

/* ------------------------------------------------------------------------- */
/* AdamW on the owner's fp32 partition (Loshchilov & Hutter, decoupled weight */
/* decay, with Kingma & Ba's bias correction; eps added after the square      */
/* root), then the 16-bit copy of the new master weight (ZeRO-2 source        */
/* walkthrough section 4.1 step 3 and section 4.3).                           */
/* ------------------------------------------------------------------------- */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm;
    int64_t step; /* t, counted from 1, after this step's increment */
} oracle_hparams;

typedef struct {
    float decay;   /* 1 - lr*wd          */
    float b1, omb1;/* beta1, 1 - beta1   */
    float b2, omb2;/* beta2, 1 - beta2   */
    float bc1, bc2;/* 1 - beta^t         */
    float lr, eps;
} oracle_adam_consts;

void oracle_adam_consts_for(const oracle_hparams* hp, oracle_adam_consts* c) {
    double t = (double)hp->step;
    c->decay = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
    c->b1 = hp->beta1;
    c->omb1 = (float)(1.0 - (double)hp->beta1);
    c->b2 = hp->beta2;
    c->omb2 = (float)(1.0 - (double)hp->beta2);
    c->bc1 = (float)(1.0 - pow((double)hp->beta1, t));
    c->bc2 = (float)(1.0 - pow((double)hp->beta2, t));
    c->lr = hp->lr;
    c->eps = hp->eps;
}

/* One AdamW step over `count` owned elements.  Does nothing when `overflow`
 * is set (the step is skipped; the caller keeps t unchanged). */
void oracle_adamw(float* master, float* exp_avg, float* exp_avg_sq, uint16_t* param16,
                  const uint16_t* red, int64_t count, int32_t dtype, float inv_scale,
                  double sumsq, uint32_t overflow, const oracle_hparams* hp) {
    if (overflow) return;
    const double* val = value_table(dtype);
    fmt16 f = fmt_of(dtype);
    oracle_adam_consts c;
    oracle_adam_consts_for(hp, &c);
    float coef = oracle_clip_coef(hp->max_grad_norm, sumsq);
    for (int64_t i = 0; i < count; ++i) {
        float g = (float)val[red[i]] * inv_scale;   /* unscale              */
        g = g * coef;                               /* clip                 */
        float p = master[i] * c.decay;              /* decoupled decay      */
        float m = c.b1 * exp_avg[i] + c.omb1 * g;   /* first moment         */
        float v = c.b2 * exp_avg_sq[i] + c.omb2 * (g * g); /* second moment */
        float mh = m / c.bc1;                       /* bias corrections     */
        float vh = v / c.bc2;
        p = p - c.lr * (mh / (sqrtf(vh) + c.eps));
        master[i] = p;
        exp_avg[i] = m;
        exp_avg_sq[i] = v;
        param16[i] = encode16((double)p, f);
    }
}

/* The same update evaluated in fp64 from the same inputs (no intermediate
 * fp32 rounding).  Used only to bound the fp32 oracle's rounding error. */
void oracle_adamw_f64(const float* master, const float* exp_avg, const float* exp_avg_sq,
                      const uint16_t* red, int64_t count, int32_t dtype, double inv_scale,
                      double coef, const oracle_hparams* hp,
                      double* master_out, double* m_out, double* v_out) {
    const double* val = value_table(dtype);
    double t = (double)hp->step;
    double lr = hp->lr, wd = hp->weight_decay, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps;
    for (int64_t i = 0; i < count; ++i) {
        double g = val[red[i]] * inv_scale * coef;
        double p = (double)master[i] * (1.0 - lr * wd);
        double m = b1 * exp_avg[i] + (1.0 - b1) * g;
        double v = b2 * exp_avg_sq[i] + (1.0 - b2) * g * g;
        double mh = m / (1.0 - pow(b1, t));
        double vh = v / (1.0 - pow(b2, t));
        master_out[i] = p - lr * (mh / (sqrt(vh) + eps));
        m_out[i] = m;
        v_out[i] = v;
    }
}

/* The 16-bit parameter copy -> fp32 master at initialisation: the master is a
 * float copy of the 16-bit partition (ZeRO-2 source walkthrough section 4.1
 * step 3).  Exact. */
void oracle_init_master(float* master, const uint16_t* param16, int64_t count, int32_t dtype) {
    const double* val = value_table(dtype);
    for (int64_t i = 0; i < count; ++i) master[i] = (float)val[param16[i]];
}

/* ------------------------------------------------------------------------- */
/* Dynamic loss scaling (wmrh.cn article section 3.1 fp16 block: loss_scale 0 */
/* means dynamic, loss_scale_window 1000, min_loss_scale 1).  On overflow the */
/* step is skipped and the scale halves, never below the minimum; after       */
/* `window` clean steps in a row it doubles.                                  */
/* ------------------------------------------------------------------------- */
typedef struct {
    double scale;
    double min_scale;
    int64_t window;
    int64_t clean;    /* clean steps since the last change */
    int64_t skipped;  /* total skipped steps                */
} oracle_scaler;

void oracle_scaler_update(oracle_scaler* s, uint32_t overflow) {
    if (overflow) {
        s->scale = fmax(s->scale / 2.0, s->min_scale);
        s->clean = 0;
        s->skipped += 1;
    } else {
        s->clean += 1;
        if (s->clean == s->window) {
            s->scale = s->scale * 2.0;
            s->clean = 0;
        }
    }
}
