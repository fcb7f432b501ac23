// zero_shard.hip -- HIP kernels and C ABI of the ZeRO-1/2 owner-shard step
// for MI355X (gfx950, CDNA4).  The ABI is documented in include/zero_shard.h.
//
// Every phase is a flat streaming pass over HBM, so the kernels are built
// around the memory system, not the ALUs:
//   * one 128-bit load or store per lane per stream (8 x 16-bit or 4 x fp32),
//     consecutive lanes on consecutive 16-byte chunks: a wave moves 1 KiB per
//     instruction per stream, fully coalesced;
//   * every stream issues all of a lane's loads for an iteration before any
//     arithmetic, so each lane keeps N x 16 B (reduce) or 7 x 16 B (AdamW) in
//     flight;
//   * non-temporal loads and stores: nothing is re-read, so nothing should
//     displace other data in L2 / the Infinity Cache;
//   * grid-stride loops over 256-thread blocks (4 wave64s), a few blocks per
//     CU; blocks are dealt round-robin to the 8 XCDs and no data is shared
//     between blocks, so no XCD-local placement is needed;
//   * reductions (norm, overflow flag) go lane -> wave (cross-lane shuffles)
//     -> block (LDS) -> one partial per block -> a single-block finalize that
//     adds the partials in a fixed order.  No floating-point atomics, so the
//     result bits depend only on the element count and alignment.
// No MFMA: nothing here is a dense contraction.
//
// Numerics (see the header for the exact per-element definition):
//   * reduce: fp64 additions in rank order, then one rounding to 16 bits.  The
//     fp64 -> 16-bit rounding is done as fp64 -> fp32 with round-to-odd,
//     then fp32 -> 16-bit to nearest-even; an intermediate format with at
//     least two more significand bits rounded to odd makes the second
//     rounding equal to a direct one (Boldo and Melquiond, "When double
//     rounding is odd", 2005).
//   * AdamW: fp32 with one rounding per operation; the library is built with
//     -ffp-contract=off and with correctly rounded fp32 division and square
//     root, so the result does not depend on instruction selection.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <tuple>

#include "zero_shard.h"

namespace {

constexpr int kThreads = 256;          // 4 wave64s per block
constexpr int kVec = 8;                // 16-bit elements per 128-bit access
constexpr int kMaxBlocks = 256 * 8;    // 256 CUs x 8 resident blocks
constexpr int kCheckMaxBlocks = 2048;  // partials of the check phase

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct RankPtrs {
    const uint16_t* p[ZERO_MAX_RANKS];
};

struct AdamConsts {
    float decay, b1, omb1, b2, omb2, bc1, bc2, lr, eps, max_norm;
};

// ---------------------------------------------------------------- memory ----
__device__ __forceinline__ u32x4 load_b128(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store_b128(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ f32x4 load_f4(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store_f4(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ uint16_t half_of(u32x4 w, int k) {
    return (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu));
}

// ------------------------------------------------------- 16-bit formats ----
template <int DT>
__device__ __forceinline__ float to_f32(uint16_t b);

template <>
__device__ __forceinline__ float to_f32<ZERO_FP16>(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);      // exact widening
}
template <>
__device__ __forceinline__ float to_f32<ZERO_BF16>(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);         // bf16 is the top half of fp32
}

template <int DT>
__device__ __forceinline__ bool nonfinite16(uint16_t b) {
    const uint16_t expo = DT == ZERO_FP16 ? 0x7C00 : 0x7F80;
    return (b & expo) == expo;
}

// fp32 -> 16 bits, round to nearest, ties to even; overflow -> inf; NaN stays NaN.
template <int DT>
__device__ __forceinline__ uint16_t from_f32(float f);

template <>
__device__ __forceinline__ uint16_t from_f32<ZERO_FP16>(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);   // hardware convert, RNE mode
}
template <>
__device__ __forceinline__ uint16_t from_f32<ZERO_BF16>(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp64 -> fp32 rounded to odd: truncate toward zero, and set the last bit if
// anything was dropped.  Infinities and NaN pass through.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
    float t = (float)d;                          // nearest-even
    double back = (double)t;
    if (back != d && __builtin_isfinite(t)) {
        uint32_t u = __float_as_uint(t);
        if (fabs(back) > fabs(d)) u -= 1u;       // was rounded away from zero
        t = __uint_as_float(u | 1u);
    }
    return t;
}

template <int DT>
__device__ __forceinline__ uint16_t round16(double d) {
    return from_f32<DT>(f64_to_f32_odd(d));
}

// -------------------------------------------------------------- init -------
template <int DT>
__global__ void __launch_bounds__(kThreads)
init_master_kernel(float* __restrict__ master, const uint16_t* __restrict__ p16, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride)
        master[i] = to_f32<DT>(p16[i]);
}

// ------------------------------------------------------------ reduce -------
template <int DT>
__device__ __forceinline__ void reduce_one(uint16_t* dst, const RankPtrs& src, int n_ranks,
                                           int64_t e) {
    double acc = (double)to_f32<DT>(src.p[0][e]);
    for (int r = 1; r < n_ranks; ++r) acc = acc + (double)to_f32<DT>(src.p[r][e]);
    dst[e] = round16<DT>(acc);
}

// Vector body over elements [head, head + 8*nvec); block 0 also does the
// head [0, head) and the tail [head + 8*nvec, count) one element per lane.
// No __restrict__: dst may be one of the sources (each element is read and
// then written by the same lane).
template <int DT, int NR>
__global__ void __launch_bounds__(kThreads)
reduce_kernel(uint16_t* dst, RankPtrs src, int64_t head, int64_t nvec, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        const int64_t e = head + i * kVec;
        u32x4 w[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) w[r] = load_b128(src.p[r] + e);
        double acc[kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) acc[k] = (double)to_f32<DT>(half_of(w[0], k));
#pragma unroll
        for (int r = 1; r < NR; ++r) {
#pragma unroll
            for (int k = 0; k < kVec; ++k) acc[k] = acc[k] + (double)to_f32<DT>(half_of(w[r], k));
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = (uint32_t)round16<DT>(acc[2 * q]) | ((uint32_t)round16<DT>(acc[2 * q + 1]) << 16);
        store_b128(dst + e, o);
    }
    if (blockIdx.x == 0) {
        const int t = threadIdx.x;
        if (t < head) reduce_one<DT>(dst, src, NR, t);
        const int64_t tail = head + nvec * kVec + t;
        if (t < kVec && tail < count) reduce_one<DT>(dst, src, NR, tail);
    }
}

// Fallback when the pointers do not share an alignment: one element per lane.
template <int DT>
__global__ void __launch_bounds__(kThreads)
reduce_scalar_kernel(uint16_t* dst, RankPtrs src, int n_ranks, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride)
        reduce_one<DT>(dst, src, n_ranks, i);
}

// ------------------------------------------------------------- check -------
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// One (sumsq, flag) partial per block.
template <int DT>
__global__ void __launch_bounds__(kThreads)
check_partial_kernel(const uint16_t* __restrict__ g, int64_t head, int64_t nvec, int64_t count,
                     int aligned, float inv_scale, double* __restrict__ part_sum,
                     uint32_t* __restrict__ part_flag) {
    const double inv = (double)inv_scale;
    double acc = 0.0;
    uint32_t bad = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (aligned) {
        for (int64_t i = tid; i < nvec; i += stride) {
            const u32x4 w = load_b128(g + head + i * kVec);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const uint16_t b = half_of(w, k);
                bad |= nonfinite16<DT>(b) ? 1u : 0u;
                const double x = (double)to_f32<DT>(b) * inv;     // exact
                acc = fma(x, x, acc);                             // x*x is exact in fp64
            }
        }
        if (blockIdx.x == 0) {
            const int t = threadIdx.x;
            int64_t e = -1;
            if (t < head) e = t;
            else if (t >= 64 && t < 64 + kVec && head + nvec * kVec + (t - 64) < count)
                e = head + nvec * kVec + (t - 64);
            if (e >= 0) {
                const uint16_t b = g[e];
                bad |= nonfinite16<DT>(b) ? 1u : 0u;
                const double x = (double)to_f32<DT>(b) * inv;
                acc = fma(x, x, acc);
            }
        }
    } else {
        for (int64_t i = tid; i < count; i += stride) {
            const uint16_t b = g[i];
            bad |= nonfinite16<DT>(b) ? 1u : 0u;
            const double x = (double)to_f32<DT>(b) * inv;
            acc = fma(x, x, acc);
        }
    }
    __shared__ double s_sum[kThreads / 64];
    __shared__ uint32_t s_flag[kThreads / 64];
    acc = wave_sum(acc);
    const uint64_t any = __ballot(bad != 0);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_sum[wave] = acc;
        s_flag[wave] = any != 0 ? 1u : 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
        uint32_t f = 0;
#pragma unroll
        for (int k = 0; k < kThreads / 64; ++k) {
            s += s_sum[k];
            f |= s_flag[k];
        }
        part_sum[blockIdx.x] = s;
        part_flag[blockIdx.x] = f;
    }
}

// Adds the partials in a fixed order and writes (or accumulates into) *res.
__global__ void __launch_bounds__(kThreads)
check_finalize_kernel(const double* __restrict__ part_sum, const uint32_t* __restrict__ part_flag,
                      int n_parts, float inv_scale, int accumulate, zero_step_result* res) {
    double s = 0.0;
    uint32_t f = 0;
    for (int k = threadIdx.x; k < n_parts; k += kThreads) {
        s += part_sum[k];
        f |= part_flag[k];
    }
    __shared__ double s_sum[kThreads / 64];
    __shared__ uint32_t s_flag[kThreads / 64];
    s = wave_sum(s);
    const uint64_t any = __ballot(f != 0);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_sum[wave] = s;
        s_flag[wave] = any != 0 ? 1u : 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double total = 0.0;
        uint32_t flag = 0;
        for (int k = 0; k < kThreads / 64; ++k) {
            total += s_sum[k];
            flag |= s_flag[k];
        }
        if (accumulate) {
            total = res->sumsq + total;
            flag |= res->overflow;
        }
        res->sumsq = total;
        res->overflow = flag;
        res->inv_scale = inv_scale;
    }
}

// ------------------------------------------------------------- AdamW -------
struct AdamElem {
    float p, m, v;
};

__device__ __forceinline__ AdamElem adam_update(const AdamConsts& c, float g, float p, float m,
                                                float v) {
    AdamElem o;
    p = p * c.decay;
    m = c.b1 * m + c.omb1 * g;
    v = c.b2 * v + c.omb2 * (g * g);
    const float mh = m / c.bc1;
    const float vh = v / c.bc2;
    o.p = p - c.lr * (mh / (sqrtf(vh) + c.eps));
    o.m = m;
    o.v = v;
    return o;
}

template <int DT>
__device__ __forceinline__ void adam_one(const AdamConsts& c, float inv, float coef, float* master,
                                         float* ma, float* va, uint16_t* p16, const uint16_t* g16,
                                         int64_t e) {
    float g = to_f32<DT>(g16[e]) * inv;
    g = g * coef;
    const AdamElem o = adam_update(c, g, master[e], ma[e], va[e]);
    master[e] = o.p;
    ma[e] = o.m;
    va[e] = o.v;
    p16[e] = from_f32<DT>(o.p);
}

template <int DT>
__global__ void __launch_bounds__(kThreads)
adamw_kernel(float* __restrict__ master, float* __restrict__ ma, float* __restrict__ va,
             uint16_t* __restrict__ p16, const uint16_t* __restrict__ g16, int64_t head,
             int64_t nvec, int64_t count, int aligned, AdamConsts c,
             const zero_step_result* __restrict__ res) {
    if (res->overflow) return;                       // skipped step: write nothing
    const float inv = res->inv_scale;
    float coef = 1.0f;
    if (c.max_norm > 0.0f) {
        const double q = (double)c.max_norm / (sqrt(res->sumsq) + 1e-6);
        if (q < 1.0) coef = (float)q;
    }
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (!aligned) {
        for (int64_t i = tid; i < count; i += stride)
            adam_one<DT>(c, inv, coef, master, ma, va, p16, g16, i);
        return;
    }
    for (int64_t i = tid; i < nvec; i += stride) {
        const int64_t e = head + i * kVec;
        const u32x4 gw = load_b128(g16 + e);
        const f32x4 p0 = load_f4(master + e), p1 = load_f4(master + e + 4);
        const f32x4 m0 = load_f4(ma + e), m1 = load_f4(ma + e + 4);
        const f32x4 v0 = load_f4(va + e), v1 = load_f4(va + e + 4);
        f32x4 po[2], mo[2], vo[2];
        uint16_t ph[kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            float g = to_f32<DT>(half_of(gw, k)) * inv;
            g = g * coef;
            const float pk = k < 4 ? p0[k & 3] : p1[k & 3];
            const float mk = k < 4 ? m0[k & 3] : m1[k & 3];
            const float vk = k < 4 ? v0[k & 3] : v1[k & 3];
            const AdamElem o = adam_update(c, g, pk, mk, vk);
            po[k >> 2][k & 3] = o.p;
            mo[k >> 2][k & 3] = o.m;
            vo[k >> 2][k & 3] = o.v;
            ph[k] = from_f32<DT>(o.p);
        }
        store_f4(master + e, po[0]);
        store_f4(master + e + 4, po[1]);
        store_f4(ma + e, mo[0]);
        store_f4(ma + e + 4, mo[1]);
        store_f4(va + e, vo[0]);
        store_f4(va + e + 4, vo[1]);
        u32x4 pw;
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = (uint32_t)ph[2 * q] | ((uint32_t)ph[2 * q + 1] << 16);
        store_b128(p16 + e, pw);
    }
    if (blockIdx.x == 0) {
        const int t = threadIdx.x;
        if (t < head) adam_one<DT>(c, inv, coef, master, ma, va, p16, g16, t);
        const int64_t tail = head + nvec * kVec + t;
        if (t < kVec && tail < count) adam_one<DT>(c, inv, coef, master, ma, va, p16, g16, tail);
    }
}

// --------------------------------------------------------------- host ------
bool valid_dtype(int32_t dt) { return dt == ZERO_FP16 || dt == ZERO_BF16; }

// Leading elements to handle one by one so that every pointer is 16-byte
// aligned for the vector body, or -1 when no such count exists.
int64_t vector_head(const void* const* p16, int n16, const void* const* p32, int n32) {
    int64_t head = -1;
    for (int k = 0; k < n16; ++k) {
        const uintptr_t a = (uintptr_t)p16[k];
        if (a & 1) return -1;
        const int64_t h = (int64_t)((16 - (a & 15)) & 15) / 2;
        if (head < 0) head = h;
        else if (head != h) return -1;
    }
    for (int k = 0; k < n32; ++k) {
        const uintptr_t a = (uintptr_t)p32[k];
        if (a & 3) return -1;
        const int64_t h = (int64_t)((16 - (a & 15)) & 15) / 4;
        if (head < 0) head = h;
        else if ((head & 3) != h) return -1;
    }
    return head < 0 ? 0 : head;
}

struct Split {
    int64_t head, nvec;
    int aligned;
};

Split split_for(int64_t head, int64_t count) {
    Split s;
    if (head < 0) {
        s.head = 0;
        s.nvec = 0;
        s.aligned = 0;
        return s;
    }
    if (head > count) head = count;
    s.head = head;
    s.nvec = (count - head) / kVec;
    s.aligned = 1;
    return s;
}

unsigned grid_for(int64_t work_items, int64_t max_blocks) {
    int64_t b = (work_items + kThreads - 1) / kThreads;
    if (b < 1) b = 1;
    if (b > max_blocks) b = max_blocks;
    return (unsigned)b;
}

// Launches `kernel` with its arguments converted to the kernel's parameter
// types and returns this launch's own status (not a stale thread-local one).
template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), unsigned grid, hipStream_t stream, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> packed(static_cast<KArgs>(args)...);
    void* ptrs[sizeof...(KArgs)];
    int i = 0;
    std::apply([&](auto&... a) { ((ptrs[i++] = (void*)&a), ...); }, packed);
    const hipError_t err =
        hipLaunchKernel((const void*)kernel, dim3(grid), dim3(kThreads), ptrs, 0, stream);
    return err == hipSuccess ? ZERO_OK : ZERO_EDEVICE;
}

template <int DT, int NR>
int launch_reduce(uint16_t* dst, const RankPtrs& src, const Split& s, int64_t count,
                  hipStream_t stream) {
    return launch(reduce_kernel<DT, NR>, grid_for(s.nvec, kMaxBlocks), stream, dst, src, s.head,
                  s.nvec, count);
}

template <int DT>
int launch_reduce_n(uint16_t* dst, const RankPtrs& src, int n, const Split& s, int64_t count,
                    hipStream_t stream) {
    switch (n) {
        case 1: return launch_reduce<DT, 1>(dst, src, s, count, stream);
        case 2: return launch_reduce<DT, 2>(dst, src, s, count, stream);
        case 3: return launch_reduce<DT, 3>(dst, src, s, count, stream);
        case 4: return launch_reduce<DT, 4>(dst, src, s, count, stream);
        case 5: return launch_reduce<DT, 5>(dst, src, s, count, stream);
        case 6: return launch_reduce<DT, 6>(dst, src, s, count, stream);
        case 7: return launch_reduce<DT, 7>(dst, src, s, count, stream);
        case 8: return launch_reduce<DT, 8>(dst, src, s, count, stream);
        case 9: return launch_reduce<DT, 9>(dst, src, s, count, stream);
        case 10: return launch_reduce<DT, 10>(dst, src, s, count, stream);
        case 11: return launch_reduce<DT, 11>(dst, src, s, count, stream);
        case 12: return launch_reduce<DT, 12>(dst, src, s, count, stream);
        case 13: return launch_reduce<DT, 13>(dst, src, s, count, stream);
        case 14: return launch_reduce<DT, 14>(dst, src, s, count, stream);
        case 15: return launch_reduce<DT, 15>(dst, src, s, count, stream);
        default: return launch_reduce<DT, 16>(dst, src, s, count, stream);
    }
}

int check_blocks(int64_t count) {
    const int64_t items = (count + kVec - 1) / kVec;
    return (int)grid_for(items, kCheckMaxBlocks);
}

}  // namespace

// ================================================================ C ABI =====
extern "C" {

const char* zero_status_str(int status) {
    switch (status) {
        case ZERO_OK: return "ok";
        case ZERO_EINVAL: return "invalid argument";
        case ZERO_ERANGE: return "size out of range";
        case ZERO_EDEVICE: return "device launch failed";
        default: return "unknown status";
    }
}

int zero_partition_layout(const int64_t* numels, int64_t n_tensors, int32_t world,
                          int32_t align_elems, int64_t* tensor_offsets, int64_t* part_begin,
                          int64_t* padded_total) {
    if (n_tensors < 0 || world < 1 || align_elems < 1 || !part_begin || !padded_total)
        return ZERO_EINVAL;
    if (n_tensors > 0 && (!numels || !tensor_offsets)) return ZERO_EINVAL;
    int64_t phi = 0;
    for (int64_t k = 0; k < n_tensors; ++k) {
        if (numels[k] < 0) return ZERO_EINVAL;
        if (__builtin_add_overflow(phi, numels[k], &phi)) return ZERO_ERANGE;
    }
    int64_t unit;
    if (__builtin_mul_overflow((int64_t)world, (int64_t)align_elems, &unit)) return ZERO_ERANGE;
    int64_t padded;
    if (__builtin_add_overflow(phi, unit - 1, &padded)) return ZERO_ERANGE;
    padded = padded / unit * unit;
    int64_t run = 0;
    for (int64_t k = 0; k < n_tensors; ++k) {
        tensor_offsets[k] = run;
        run += numels[k];
    }
    const int64_t part = padded / world;
    for (int32_t p = 0; p <= world; ++p) part_begin[p] = part * p;
    *padded_total = padded;
    return ZERO_OK;
}

int zero_bucket_layout(const int64_t* numels, int64_t n_tensors, int64_t bucket_cap,
                       int64_t* bucket_first, int64_t* n_buckets) {
    if (n_tensors < 0 || bucket_cap < 1 || !bucket_first || !n_buckets) return ZERO_EINVAL;
    if (n_tensors > 0 && !numels) return ZERO_EINVAL;
    int64_t nb = 0;
    int64_t room = 0;       // free elements left in the open bucket
    bool open_empty = true;
    for (int64_t k = 0; k < n_tensors; ++k) {
        const int64_t n = numels[k];
        if (n < 0) return ZERO_EINVAL;
        if (k == 0 || (!open_empty && n > room)) {
            bucket_first[nb++] = k;
            room = bucket_cap;
            open_empty = true;
        }
        room -= n;                 // may go negative for an oversized tensor
        if (n > 0) open_empty = false;
    }
    bucket_first[nb] = n_tensors;
    *n_buckets = nb;
    return ZERO_OK;
}

int zero_memory_bytes(int32_t stage, int64_t numel_total, int64_t padded_total, int32_t world,
                      int64_t* bytes_out) {
    if (stage < 0 || stage > 3 || world < 1 || numel_total < 0 || !bytes_out) return ZERO_EINVAL;
    if (padded_total < numel_total || padded_total % world != 0) return ZERO_EINVAL;
    const int64_t part = padded_total / world;
    const int64_t params = stage >= 3 ? part : numel_total;
    const int64_t grads = stage >= 2 ? part : numel_total;
    const int64_t optim = stage >= 1 ? part : numel_total;
    int64_t a, b, c, t;
    if (__builtin_mul_overflow(params, (int64_t)2, &a) ||
        __builtin_mul_overflow(grads, (int64_t)2, &b) ||
        __builtin_mul_overflow(optim, (int64_t)12, &c) || __builtin_add_overflow(a, b, &t) ||
        __builtin_add_overflow(t, c, &t))
        return ZERO_ERANGE;
    *bytes_out = t;
    return ZERO_OK;
}

int zero_loss_scaler_update(zero_loss_scaler* s, uint32_t overflow) {
    if (!s || s->window < 1) return ZERO_EINVAL;
    if (overflow) {
        const double half = s->scale * 0.5;
        s->scale = half > s->min_scale ? half : s->min_scale;
        s->clean = 0;
        s->skipped += 1;
    } else {
        s->clean += 1;
        if (s->clean >= s->window) {
            s->scale = s->scale * 2.0;
            s->clean = 0;
        }
    }
    return ZERO_OK;
}

int zero_init_master(float* master, const void* param16, int64_t count, int32_t dtype,
                     hipStream_t stream) {
    if (count < 0 || !valid_dtype(dtype)) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    if (!master || !param16) return ZERO_EINVAL;
    const unsigned grid = grid_for(count, kMaxBlocks);
    const uint16_t* p = (const uint16_t*)param16;
    return dtype == ZERO_FP16 ? launch(init_master_kernel<ZERO_FP16>, grid, stream, master, p, count)
                              : launch(init_master_kernel<ZERO_BF16>, grid, stream, master, p, count);
}

int zero_reduce_owned(void* dst, const void* const* srcs, int32_t n_ranks, int64_t count,
                      int32_t dtype, hipStream_t stream) {
    if (count < 0 || n_ranks < 1 || n_ranks > ZERO_MAX_RANKS || !valid_dtype(dtype) || !srcs)
        return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    if (!dst) return ZERO_EINVAL;
    RankPtrs rp;
    const void* all16[ZERO_MAX_RANKS + 1];
    for (int r = 0; r < ZERO_MAX_RANKS; ++r) rp.p[r] = nullptr;
    for (int r = 0; r < n_ranks; ++r) {
        if (!srcs[r]) return ZERO_EINVAL;
        rp.p[r] = (const uint16_t*)srcs[r];
        all16[r] = srcs[r];
    }
    all16[n_ranks] = dst;
    const Split s = split_for(vector_head(all16, n_ranks + 1, nullptr, 0), count);
    uint16_t* d = (uint16_t*)dst;
    if (!s.aligned) {
        const unsigned grid = grid_for(count, kMaxBlocks);
        return dtype == ZERO_FP16
                   ? launch(reduce_scalar_kernel<ZERO_FP16>, grid, stream, d, rp, n_ranks, count)
                   : launch(reduce_scalar_kernel<ZERO_BF16>, grid, stream, d, rp, n_ranks, count);
    }
    return dtype == ZERO_FP16 ? launch_reduce_n<ZERO_FP16>(d, rp, n_ranks, s, count, stream)
                              : launch_reduce_n<ZERO_BF16>(d, rp, n_ranks, s, count, stream);
}

size_t zero_check_workspace_bytes(int64_t count) {
    if (count < 0) count = 0;
    return (size_t)check_blocks(count) * (sizeof(double) + sizeof(uint32_t));
}

int zero_unscale_check_norm(const void* grad16, int64_t count, int32_t dtype, float inv_scale,
                            zero_step_result* res, void* workspace, size_t workspace_bytes,
                            int32_t accumulate, hipStream_t stream) {
    if (count < 0 || !valid_dtype(dtype) || !res || !workspace) return ZERO_EINVAL;
    if (count > 0 && !grad16) return ZERO_EINVAL;
    if (workspace_bytes < zero_check_workspace_bytes(count)) return ZERO_EINVAL;
    if (((uintptr_t)workspace & 7) != 0) return ZERO_EINVAL;
    const int blocks = check_blocks(count);
    double* part_sum = (double*)workspace;
    uint32_t* part_flag = (uint32_t*)(part_sum + blocks);
    const void* p = grad16;
    const Split s = split_for(vector_head(&p, 1, nullptr, 0), count);
    const uint16_t* g = (const uint16_t*)grad16;
    const int rc =
        dtype == ZERO_FP16
            ? launch(check_partial_kernel<ZERO_FP16>, (unsigned)blocks, stream, g, s.head, s.nvec,
                     count, s.aligned, inv_scale, part_sum, part_flag)
            : launch(check_partial_kernel<ZERO_BF16>, (unsigned)blocks, stream, g, s.head, s.nvec,
                     count, s.aligned, inv_scale, part_sum, part_flag);
    if (rc != ZERO_OK) return rc;
    return launch(check_finalize_kernel, 1u, stream, part_sum, part_flag, blocks, inv_scale,
                  (int)(accumulate != 0), res);
}

int zero_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                    const void* grad16, int64_t count, int32_t dtype,
                    const zero_adamw_hparams* hp, const zero_step_result* res,
                    hipStream_t stream) {
    if (count < 0 || !valid_dtype(dtype) || !hp || !res || hp->step < 1) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !param16 || !grad16) return ZERO_EINVAL;
    AdamConsts c;
    const double t = (double)hp->step;
    c.decay = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
    c.b1 = hp->beta1;
    c.omb1 = (float)(1.0 - (double)hp->beta1);
    c.b2 = hp->beta2;
    c.omb2 = (float)(1.0 - (double)hp->beta2);
    c.bc1 = (float)(1.0 - pow((double)hp->beta1, t));
    c.bc2 = (float)(1.0 - pow((double)hp->beta2, t));
    c.lr = hp->lr;
    c.eps = hp->eps;
    c.max_norm = hp->max_grad_norm;
    const void* p16s[2] = {param16, grad16};
    const void* p32s[3] = {master, exp_avg, exp_avg_sq};
    const Split s = split_for(vector_head(p16s, 2, p32s, 3), count);
    const unsigned grid = grid_for(s.aligned ? s.nvec : count, kMaxBlocks);
    uint16_t* p16 = (uint16_t*)param16;
    const uint16_t* g16 = (const uint16_t*)grad16;
    return dtype == ZERO_FP16
               ? launch(adamw_kernel<ZERO_FP16>, grid, stream, master, exp_avg, exp_avg_sq, p16,
                        g16, s.head, s.nvec, count, s.aligned, c, res)
               : launch(adamw_kernel<ZERO_BF16>, grid, stream, master, exp_avg, exp_avg_sq, p16,
                        g16, s.head, s.nvec, count, s.aligned, c, res);
}

}  // extern "C"
