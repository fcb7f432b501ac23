// zero_shard.hip -- HIP kernels and C ABI of the ZeRO-1/2 owner-shard step
// for MI355X (gfx950, CDNA4).  The ABI is documented in include/zero_shard.h.
//
// Every phase is a flat streaming pass over HBM, so the kernels are built
// around the memory system, not the ALUs:
//   * a lane tile is 8 consecutive elements: one 128-bit load per 16-bit
//     stream and two per fp32 stream; consecutive lanes own consecutive
//     tiles, so a wave64 moves 1 KiB (16-bit) or 2 KiB (fp32) per stream per
//     instruction, fully coalesced;
//   * one 256-lane block per 1 (AdamW, check) or 2 (reduce) block-wide rows
//     of lane tiles, no grid-stride loop: the hardware dispatcher keeps every
//     CU of the 8 XCDs fed with short-lived blocks and the whole chip sweeps
//     the buffers front to back.  On MI355X this beats a persistent
//     grid-stride grid by 15-25% for every stream mix measured here;
//   * all of a lane's loads are issued before any arithmetic;
//   * the kernels with many concurrent streams (AdamW: 4 read + 4 write;
//     the reduce: N + 1) cap the blocks resident per CU with dynamic LDS:
//     fewer waves in flight keep fewer DRAM rows open at once, and enough
//     bytes stay in flight to cover the latency (AdamW 6.10 -> 6.37 TB/s on
//     the LLaMA-70B-shaped shard, where a math-free twin of its stream mix
//     peaks at 6.35);
//   * data read once (rank gradients, the reduced gradient in AdamW) is
//     loaded non-temporally, and the reduce stores non-temporally; AdamW
//     updates master / m / v in place with plain accesses, which measured
//     faster;
//   * reductions (norm, overflow flag) go lane -> wave (cross-lane shuffles)
//     -> block (LDS) -> one partial per block -> fold passes of 2048 partials
//     per block -> one finalize block.  No floating-point atomics: the result
//     bits depend only on the element count and the pointers' alignment.
// No MFMA: nothing here is a dense contraction.
//
// Numerics (the header gives the per-element definitions):
//   * reduce: fp32 additions in rank order starting from +0, then one rounding
//     to 16 bits, nearest-even (hardware convert for binary16, integer
//     rounding of the upper half for bfloat16);
//   * check: the unscaled value is the fp32 product float(v) * inv_scale; its
//     square is exact in fp64 and summed in fp64;
//   * AdamW: fp32 with one rounding per operation; the library is built with
//     -ffp-contract=off and with correctly rounded fp32 division and square
//     root, so the result does not depend on instruction selection.

#include <math.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "zero_common.h"

namespace {

struct RankPtrs {
    const uint16_t* p[ZERO_MAX_RANKS];
};

struct AdamConsts {
    float decay, b1, omb1, b2, omb2, bc1, bc2, lr, eps, max_norm;
};

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

// --------------------------------------------------- block reductions -----
// Sum of `s` and OR of `f` over the block, in a fixed order; valid in thread 0.
__device__ __forceinline__ void block_sum_or(double& s, uint32_t& f) {
    __shared__ double s_sum[kThreads / 64];
    __shared__ uint32_t s_flag[kThreads / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const uint64_t any = __ballot(f != 0);
    if ((threadIdx.x & 63) == 0) {
        s_sum[threadIdx.x >> 6] = s;
        s_flag[threadIdx.x >> 6] = any != 0 ? 1u : 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        s = 0.0;
        f = 0;
#pragma unroll
        for (int k = 0; k < kThreads / 64; ++k) {
            s += s_sum[k];
            f |= s_flag[k];
        }
    }
}

// Accumulates one checked 16-bit value into (sq, bad): the unscaled value is
// the fp32 product float(b) * inv; its square is exact in fp64.
template <int DT>
__device__ __forceinline__ void check_acc(uint16_t b, float inv, double& sq, uint32_t& bad) {
    bad |= nonfinite16<DT>(b) ? 1u : 0u;
    const double x = (double)(to_f32<DT>(b) * inv);
    sq = fma(x, x, sq);                             // x*x is exact in fp64
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
__device__ __forceinline__ uint16_t reduce_one(const RankPtrs& src, int n_ranks, int64_t e) {
    float acc = 0.0f;
    for (int r = 0; r < n_ranks; ++r) acc = acc + to_f32<DT>(src.p[r][e]);
    return from_f32<DT>(acc);
}

// One lane tile of the reduce: the NR ranks' 128-bit words w[] of 8
// elements, fp32 additions in rank order from +0 (0 + -0 is +0, so the first
// addition is kept), one rounding to 16 bits, stored at d; with CHECK the
// reduced values also go into (sq, bad).
template <int DT, int NR, bool CHECK>
__device__ __forceinline__ void reduce_tile(const u32x4 (&w)[NR], uint16_t* d, float inv, double& sq,
                                            uint32_t& bad) {
    float acc[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) acc[k] = 0.0f + to_f32<DT>(half_of(w[0], k));
#pragma unroll
    for (int r = 1; r < NR; ++r) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) acc[k] = acc[k] + to_f32<DT>(half_of(w[r], k));
    }
    uint16_t h[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        h[k] = from_f32<DT>(acc[k]);
        if (CHECK) check_acc<DT>(h[k], inv, sq, bad);
    }
    store_nt(d, pack8(h));
}

// Lane tiles per lane in the reduce, and resident blocks per CU for NR
// ranks: about 32 of a lane's 128-bit loads in flight per SIMD-slot whatever
// the rank count (measured on MI355X: 8 ranks 5.83 -> 5.92-6.11 TB/s with
// 2 blocks per CU, 16 ranks 5.70 -> 5.88 TB/s with 1).
constexpr int kReduceTiles = 2;
constexpr int reduce_blocks_per_cu(int nr) { return nr >= 16 ? 1 : (16 / nr > 8 ? 8 : 16 / nr); }
// Elements of one reduce block, and the rank count whose whole blocks stage
// their rank data in LDS (reduce_block_lds): 8 ranks x 8 KiB = 64 KiB per
// block, two blocks per CU.  On MI355X that ran 4.4-4.9 % faster than
// loading into registers at the LLaMA-7B shard size and 1.8-2.0 % at the
// 70B size (same placements, A/B); at 1-6 ranks it made no difference and at
// 12-16 ranks (one block per CU) it was 7 % slower.
constexpr int kReduceBlockElems = kReduceTiles * kTile;
constexpr int kLdsRanks = 8;
constexpr unsigned kReduceLdsBytes = kLdsRanks * kReduceBlockElems * 2;
// Dynamic LDS of a reduce launch over nr ranks: the occupancy cap, or for
// the LDS-staged rank count its staging buffer (64 KiB, which leaves room for
// the same two blocks per CU).
inline unsigned reduce_lds(int nr) {
    const unsigned cap = lds_for_blocks(reduce_blocks_per_cu(nr));
    return nr == kLdsRanks && kReduceLdsBytes > cap ? kReduceLdsBytes : cap;
}
static_assert(2 * kReduceLdsBytes <= kLdsPerCU && 3 * kReduceLdsBytes > kLdsPerCU,
              "the 8-rank staging buffer keeps two blocks per CU");

// Reduce of NR ranks; with CHECK also the overflow flag and squared norm of
// the reduced values, one partial per block.  Block b owns kReduceTiles
// block-wide rows of lane tiles; a lane issues all its loads (kReduceTiles
// x NR 128-bit words) before any arithmetic.  No __restrict__ on dst / src:
// dst may be one of the sources (every element is read, then written, by
// the same lane).
// A whole block of the 8-rank reduce with the rank data staged in LDS: each
// wave copies two 1 KiB chunks of every rank straight into LDS (rank-major
// issue order), the block waits for all of them, then every lane reduces the
// same two lane tiles as in the register path (elements 8t and 2048 + 8t of
// the block for lane t), in the same order, so the sums, the stored values
// and the block's partial are bit-identical to that path.
template <int DT, bool CHECK>
__device__ __forceinline__ void reduce_block_lds(uint16_t* dst, const RankPtrs& src, int64_t e0,
                                                 float& inv, const zero_step_control* ctl,
                                                 double& sq, uint32_t& bad) {
    extern __shared__ __attribute__((aligned(16))) char stage[];   // kReduceLdsBytes
    constexpr int kChunk = 512;                                     // elements per wave copy
    constexpr int kChunks = kReduceBlockElems / kChunk;             // per rank
    constexpr int kWaves = kThreads / 64;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < kLdsRanks; ++r)
#pragma unroll
        for (int j = 0; j < kChunks / kWaves; ++j) {
            const int ch = w + kWaves * j;
            load_to_lds<true>(src.p[r] + e0 + ch * kChunk + lane * kVec,
                              stage + (r * kChunks + ch) * (kChunk * 2));
        }
    if (CHECK && ctl) inv = ctl->inv_scale;         // while the copies are in flight
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kReduceTiles; ++t) {
        const int q = t * kThreads + threadIdx.x;   // lane tile within the block
        u32x4 w8[kLdsRanks];
#pragma unroll
        for (int r = 0; r < kLdsRanks; ++r)
            w8[r] = *reinterpret_cast<const u32x4*>(stage + r * (kReduceBlockElems * 2) + q * 16);
        reduce_tile<DT, kLdsRanks, CHECK>(w8, dst + e0 + q * kVec, inv, sq, bad);
    }
}

template <int DT, int NR, bool CHECK>
__device__ __forceinline__ void reduce_block(uint16_t* dst, const RankPtrs& src, const Split& s,
                                             float inv, const zero_step_control* ctl,
                                             double* part_sum, uint32_t* part_flag) {
    double sq = 0.0;
    uint32_t bad = 0;
    const int64_t blk = block_id(s);
    // With device step control the unscale factor is read from ctl after the
    // rank loads are issued: read before them, its scalar-load latency would
    // sit in front of every block's HBM loads.
    if (s.aligned) {
        if (NR == kLdsRanks && (blk + 1) * (kReduceTiles * kThreads) <= s.nvec) {  // whole block
            reduce_block_lds<DT, CHECK>(dst, src, s.head + blk * kReduceBlockElems, inv, ctl, sq,
                                        bad);
        } else if (lane_tile<kReduceTiles>(s, kReduceTiles - 1) < s.nvec) {   // every row in range
            u32x4 w[kReduceTiles][NR];
#pragma unroll
            for (int t = 0; t < kReduceTiles; ++t) {
                const int64_t e = s.head + lane_tile<kReduceTiles>(s, t) * kVec;
#pragma unroll
                for (int r = 0; r < NR; ++r) w[t][r] = load_nt(src.p[r] + e);
            }
            if (CHECK && ctl) inv = ctl->inv_scale;
#pragma unroll
            for (int t = 0; t < kReduceTiles; ++t)
                reduce_tile<DT, NR, CHECK>(w[t], dst + s.head + lane_tile<kReduceTiles>(s, t) * kVec,
                                           inv, sq, bad);
        } else {
#pragma unroll
            for (int t = 0; t < kReduceTiles; ++t) {
                const int64_t i = lane_tile<kReduceTiles>(s, t);
                if (i < s.nvec) {
                    const int64_t e = s.head + i * kVec;
                    u32x4 w[NR];
#pragma unroll
                    for (int r = 0; r < NR; ++r) w[r] = load_nt(src.p[r] + e);
                    if (CHECK && ctl) inv = ctl->inv_scale;
                    reduce_tile<DT, NR, CHECK>(w, dst + e, inv, sq, bad);
                }
            }
        }
        if (blk == 0) {
            const int t = threadIdx.x;
            int64_t e = -1;
            if (t < s.head) e = t;
            else if (t >= 64 && t < 64 + kVec && s.head + s.nvec * kVec + (t - 64) < s.count)
                e = s.head + s.nvec * kVec + (t - 64);
            if (e >= 0) {
                if (CHECK && ctl) inv = ctl->inv_scale;
                const uint16_t h = reduce_one<DT>(src, NR, e);
                dst[e] = h;
                if (CHECK) check_acc<DT>(h, inv, sq, bad);
            }
        }
    } else {
        if (CHECK && ctl) inv = ctl->inv_scale;
        for (int t = 0; t < kReduceTiles; ++t) {
            const int64_t i = lane_tile<kReduceTiles>(s, t);
            for (int64_t e = i * kVec; e < (i + 1) * kVec && e < s.count; ++e) {
                const uint16_t h = reduce_one<DT>(src, NR, e);
                dst[e] = h;
                if (CHECK) check_acc<DT>(h, inv, sq, bad);
            }
        }
    }
    if (CHECK) {
        block_sum_or(sq, bad);
        if (threadIdx.x == 0) {
            part_sum[blk] = sq;
            part_flag[blk] = bad;
        }
    }
}

template <int DT, int NR, bool CHECK>
__global__ void __launch_bounds__(kThreads)
reduce_kernel(uint16_t* dst, RankPtrs src, Split s, float inv, const zero_step_control* ctl,
              double* part_sum, uint32_t* part_flag) {
    reduce_block<DT, NR, CHECK>(dst, src, s, inv, ctl, part_sum, part_flag);
}

// ------------------------------------------------------------- check -------
template <int DT>
__global__ void __launch_bounds__(kThreads)
check_kernel(const uint16_t* __restrict__ g, Split s, float inv, const zero_step_control* ctl,
             double* __restrict__ part_sum, uint32_t* __restrict__ part_flag) {
    double sq = 0.0;
    uint32_t bad = 0;
    const int64_t i = lane_tile(s);
    if (s.aligned) {
        if (i < s.nvec) {
            const u32x4 w = load_nt(g + s.head + i * kVec);
            if (ctl) inv = ctl->inv_scale;              // after the load is issued
#pragma unroll
            for (int k = 0; k < kVec; ++k) check_acc<DT>(half_of(w, k), inv, sq, bad);
        }
        if (block_id(s) == 0) {
            const int t = threadIdx.x;
            if (ctl) inv = ctl->inv_scale;
            if (t < s.head) check_acc<DT>(g[t], inv, sq, bad);
            else if (t >= 64 && t < 64 + kVec && s.head + s.nvec * kVec + (t - 64) < s.count)
                check_acc<DT>(g[s.head + s.nvec * kVec + (t - 64)], inv, sq, bad);
        }
    } else {
        if (ctl) inv = ctl->inv_scale;
        for (int64_t e = i * kVec; e < (i + 1) * kVec && e < s.count; ++e)
            check_acc<DT>(g[e], inv, sq, bad);
    }
    block_sum_or(sq, bad);
    if (threadIdx.x == 0) {
        part_sum[block_id(s)] = sq;
        part_flag[block_id(s)] = bad;
    }
}

// One fold pass: block b adds partials [b*kFold, (b+1)*kFold) in a fixed order.
__global__ void __launch_bounds__(kThreads)
fold_kernel(const double* __restrict__ in_sum, const uint32_t* __restrict__ in_flag, int64_t n,
            double* __restrict__ out_sum, uint32_t* __restrict__ out_flag) {
    double s = 0.0;
    uint32_t f = 0;
    const int64_t base = (int64_t)blockIdx.x * kFold;
#pragma unroll
    for (int k = 0; k < kFold / kThreads; ++k) {
        const int64_t j = base + k * kThreads + threadIdx.x;
        if (j < n) {
            s += in_sum[j];
            f |= in_flag[j];
        }
    }
    block_sum_or(s, f);
    if (threadIdx.x == 0) {
        out_sum[blockIdx.x] = s;
        out_flag[blockIdx.x] = f;
    }
}

// Last pass (n <= kFinal partials): writes, or accumulates into, *res.
// Thread k adds partials k, k + 256, ... in order.  Taking up to 16384
// partials here (about 200 KB, a few microseconds for one block) spares the
// fold launch for every call of up to 67e6 elements (e.g. one bucket window
// of one owner).
__global__ void __launch_bounds__(kThreads)
finalize_kernel(const double* __restrict__ in_sum, const uint32_t* __restrict__ in_flag, int64_t n,
                float inv_scale, const zero_step_control* ctl, int accumulate,
                zero_step_result* res) {
    double s = 0.0;
    uint32_t f = 0;
    for (int64_t j = threadIdx.x; j < n; j += kThreads) {
        s += in_sum[j];
        f |= in_flag[j];
    }
    block_sum_or(s, f);
    if (threadIdx.x == 0) {
        if (accumulate) {
            s = res->sumsq + s;
            f |= res->overflow;
        }
        res->sumsq = s;
        res->overflow = f;
        res->inv_scale = ctl ? ctl->inv_scale : inv_scale;
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

// Clip factor from the global squared norm: max_norm / (norm + 1e-6) when
// that is below 1, else 1; off when max_norm <= 0.  fp64, rounded once.
__device__ __forceinline__ float clip_coef(const AdamConsts& c, const zero_step_result* res) {
    float coef = 1.0f;
    if (c.max_norm > 0.0f) {
        const double q = (double)c.max_norm / (sqrt(res->sumsq) + 1e-6);
        if (q < 1.0) coef = (float)q;
    }
    return coef;
}

// The step's constants: the host's, or with device step control the betas
// and bias corrections from ctl (1 - beta is exact in fp64, rounded once).
__device__ __forceinline__ AdamConsts step_consts(AdamConsts c, const zero_step_control* ctl) {
    if (ctl) {
        c.b1 = ctl->beta1;
        c.omb1 = (float)(1.0 - (double)c.b1);
        c.b2 = ctl->beta2;
        c.omb2 = (float)(1.0 - (double)c.b2);
        c.bc1 = ctl->bc1;
        c.bc2 = ctl->bc2;
    }
    return c;
}

// AdamW over NQ element quads of one lane (NQ = 1 or 2): quad q holds the
// 4 consecutive elements at e[q].  Every load is issued before any
// arithmetic; the clip factor (and, with device step control, the step's
// constants) are read after the loads, so the fp64 square root and division
// overlap the HBM latency (computed before the loads they cost ~3% at 2
// blocks per CU).
template <int DT, int NQ>
__device__ __forceinline__ void adam_quads(const AdamConsts& c0, const zero_step_control* ctl,
                                           const zero_step_result* res, float* master, float* ma,
                                           float* va, uint16_t* p16, const uint16_t* g16,
                                           const int64_t (&e)[NQ]) {
    u32x2 gw[NQ];
    f32x4 p[NQ], m[NQ], v[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        gw[q] = load_nt_b64(g16 + e[q]);            // read once: non-temporal
        p[q] = load_f4(master + e[q]);
        m[q] = load_f4(ma + e[q]);
        v[q] = load_f4(va + e[q]);
    }
    const AdamConsts c = step_consts(c0, ctl);
    const float inv = res->inv_scale, coef = clip_coef(c, res);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        uint16_t ph[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float g = to_f32<DT>(half_of2(gw[q], k)) * inv;
            g = g * coef;
            const AdamElem o = adam_update(c, g, p[q][k], m[q][k], v[q][k]);
            p[q][k] = o.p;
            m[q][k] = o.m;
            v[q][k] = o.v;
            ph[k] = from_f32<DT>(o.p);
        }
        store_f4(master + e[q], p[q]);
        store_f4(ma + e[q], m[q]);
        store_f4(va + e[q], v[q]);
        store_nt_b64(p16 + e[q], pack4(ph));         // written once: non-temporal
    }
}

// A whole AdamW block with each wave's inputs staged in LDS: wave w owns the
// 512 consecutive elements at e0 + 512 w and copies its gradient (1 KiB) and
// master / m / v (2 KiB each) straight into its own 7 KiB of LDS, then its
// lane l updates the quads at 4l and 256 + 4l of those elements.  No block
// barrier: a wave reads only what it copied, once its own copies have
// landed, so the waves of a block run independently.  On MI355X this ran
// 0.3-1.8 % faster than the register path (LLaMA-7B and 70B shard sizes,
// several layouts, A/B); the per-element arithmetic is the same, so the
// results are bit-identical.
constexpr int kAdamWaveElems = kTile / (kThreads / 64);        // 512
constexpr int kAdamWaveBytes = kAdamWaveElems * (2 + 3 * 4);   // 7 KiB

template <int DT>
__device__ __forceinline__ void adam_block_lds(const AdamConsts& c0, const zero_step_control* ctl,
                                               const zero_step_result* res, float* master,
                                               float* ma, float* va, uint16_t* p16,
                                               const uint16_t* g16, int64_t e0) {
    extern __shared__ __attribute__((aligned(16))) char stage[];   // kThreads / 64 waves
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t e = e0 + (int64_t)w * kAdamWaveElems;
    char* lg = stage + w * kAdamWaveBytes;                         // 16-bit gradient, 1 KiB
    char* lp = lg + kAdamWaveElems * 2;                            // master, 2 KiB
    char* lm = lp + kAdamWaveElems * 4;                            // m
    char* lv = lm + kAdamWaveElems * 4;                            // v
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t o = e + j * 256 + lane * 4;
        load_to_lds<false>(master + o, lp + j * 1024);
        load_to_lds<false>(ma + o, lm + j * 1024);
        load_to_lds<false>(va + o, lv + j * 1024);
    }
    // the gradient after the state (on MI355X 0.5-1.0 % faster than first,
    // at the LLaMA-7B and 70B shard sizes and several bases, A/B)
    load_to_lds<true>(g16 + e + lane * 8, lg);                    // read once: non-temporal
    // the step's scalars while the copies are in flight
    const AdamConsts c = step_consts(c0, ctl);
    const float inv = res->inv_scale, coef = clip_coef(c, res);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = lane + 64 * j;                               // quad of the wave's elements
        const u32x2 gw = *reinterpret_cast<const u32x2*>(lg + q * 8);
        f32x4 p = *reinterpret_cast<const f32x4*>(lp + q * 16);
        f32x4 m = *reinterpret_cast<const f32x4*>(lm + q * 16);
        f32x4 v = *reinterpret_cast<const f32x4*>(lv + q * 16);
        uint16_t ph[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float g = to_f32<DT>(half_of2(gw, k)) * inv;
            g = g * coef;
            const AdamElem o = adam_update(c, g, p[k], m[k], v[k]);
            p[k] = o.p;
            m[k] = o.m;
            v[k] = o.v;
            ph[k] = from_f32<DT>(o.p);
        }
        const int64_t x = e + 4 * q;
        store_f4(master + x, p);
        store_f4(ma + x, m);
        store_f4(va + x, v);
        store_nt_b64(p16 + x, pack4(ph));                          // written once: non-temporal
    }
}

// Blocks that lie wholly inside the vector body take adam_block_lds.  In the
// last, partial block lane l takes the quads at 4l and kTile/2 + 4l of the
// block's kTile elements, so every fp32 access instruction of a wave covers
// 1 KiB contiguously and the 16-bit streams 512 B.
template <int DT>
__device__ __forceinline__ void adamw_block(float* __restrict__ master, float* __restrict__ ma,
                                            float* __restrict__ va, uint16_t* __restrict__ p16,
                                            const uint16_t* __restrict__ g16, const Split& s,
                                            const AdamConsts& c0,
                                            const zero_step_control* __restrict__ ctl,
                                            const zero_step_result* __restrict__ res) {
    if (res->overflow) return;                       // skipped step: write nothing
    if (!s.aligned) {
        const int64_t i = lane_tile(s);
        const AdamConsts c = step_consts(c0, ctl);
        const float inv = res->inv_scale, coef = clip_coef(c, res);
        for (int64_t e = i * kVec; e < (i + 1) * kVec && e < s.count; ++e)
            adam_one<DT>(c, inv, coef, master, ma, va, p16, g16, e);
        return;
    }
    // quads are offsets into the vector body [head, head + 8 nvec), whose
    // length is a multiple of 8: a quad lies wholly inside it or outside
    const int64_t body = s.nvec * kVec;
    const int64_t b0 = block_id(s) * kTile;
    const int64_t o0 = b0 + 4 * threadIdx.x;
    const int64_t o1 = o0 + kTile / 2;
    if (b0 + kTile <= body) {
        adam_block_lds<DT>(c0, ctl, res, master, ma, va, p16, g16, s.head + b0);
    } else if (o1 < body) {
        const int64_t e[2] = {s.head + o0, s.head + o1};
        adam_quads<DT, 2>(c0, ctl, res, master, ma, va, p16, g16, e);
    } else if (o0 < body) {
        const int64_t e[1] = {s.head + o0};
        adam_quads<DT, 1>(c0, ctl, res, master, ma, va, p16, g16, e);
    }
    if (block_id(s) == 0) {
        const AdamConsts c = step_consts(c0, ctl);
        const float inv = res->inv_scale, coef = clip_coef(c, res);
        const int t = threadIdx.x;
        if (t < s.head) adam_one<DT>(c, inv, coef, master, ma, va, p16, g16, t);
        else if (t >= 64 && t < 64 + kVec && s.head + body + (t - 64) < s.count)
            adam_one<DT>(c, inv, coef, master, ma, va, p16, g16, s.head + body + (t - 64));
    }
}

template <int DT>
__global__ void __launch_bounds__(kThreads)
adamw_kernel(float* __restrict__ master, float* __restrict__ ma, float* __restrict__ va,
             uint16_t* __restrict__ p16, const uint16_t* __restrict__ g16, Split s, AdamConsts c0,
             const zero_step_control* __restrict__ ctl, const zero_step_result* __restrict__ res) {
    adamw_block<DT>(master, ma, va, p16, g16, s, c0, ctl, res);
}

// ------------------------------------------------- device step control ---
// One thread ends a step: the loss-scale rule of zero_loss_scaler_update, t
// advanced on applied steps, and the next step's derived scalars.
__global__ void __launch_bounds__(64)
control_update_kernel(zero_step_control* ctl, const zero_step_result* res) {
    if (threadIdx.x != 0) return;
    zero_step_control c = *ctl;
    if (res->overflow) {
        const double half = c.scale * 0.5;
        c.scale = half > c.min_scale ? half : c.min_scale;
        c.clean = 0;
        c.skipped += 1;
    } else {
        c.t += 1;
        c.clean += 1;
        if (c.clean >= c.window) {
            c.scale = c.scale * 2.0;
            c.clean = 0;
        }
    }
    c.inv_scale = (float)(1.0 / (c.scale * (double)c.divisor));
    c.bc1 = (float)(1.0 - pow((double)c.beta1, (double)(c.t + 1)));
    c.bc2 = (float)(1.0 - pow((double)c.beta2, (double)(c.t + 1)));
    *ctl = c;
}

// --------------------------------------------------------------- host ------
// Workspace layout: fold levels of (double sums, uint32 flags), each level
// 8-byte aligned; level 0 has one partial per tile block.
struct Levels {
    int n;
    int64_t parts[8];
    size_t sum_off[8], flag_off[8];
    size_t bytes;
};

Levels levels_for(int64_t blocks) {
    Levels L;
    L.n = 0;
    size_t off = 0;
    int64_t n = blocks;
    while (true) {
        L.parts[L.n] = n;
        L.sum_off[L.n] = off;
        off += (size_t)n * sizeof(double);
        L.flag_off[L.n] = off;
        off += ((size_t)n * sizeof(uint32_t) + 7) & ~(size_t)7;
        L.n += 1;
        if (n <= kFinal) break;
        n = (n + kFold - 1) / kFold;
    }
    L.bytes = off;
    return L;
}

unsigned stream_grid(int64_t items) {
    int64_t b = (items + kThreads - 1) / kThreads;
    if (b < 1) b = 1;
    if (b > kMaxStreamBlocks) b = kMaxStreamBlocks;
    return (unsigned)b;
}

// Folds the level-0 partials into *res: fold passes, then the finalize block.
int fold_into(char* ws, const Levels& L, float inv_scale, const zero_step_control* ctl,
              int32_t accumulate, zero_step_result* res, hipStream_t stream) {
    for (int l = 0; l + 1 < L.n; ++l) {
        const int rc = launch(fold_kernel, L.parts[l + 1], 0, stream, (const double*)(ws + L.sum_off[l]),
                              (const uint32_t*)(ws + L.flag_off[l]), L.parts[l],
                              (double*)(ws + L.sum_off[l + 1]), (uint32_t*)(ws + L.flag_off[l + 1]));
        if (rc != ZERO_OK) return rc;
    }
    const int last = L.n - 1;
    return launch(finalize_kernel, 1, 0, stream, (const double*)(ws + L.sum_off[last]),
                  (const uint32_t*)(ws + L.flag_off[last]), L.parts[last], inv_scale, ctl,
                  (int)(accumulate != 0), res);
}

template <int DT, bool CHECK>
int launch_reduce_n(uint16_t* dst, const RankPtrs& src, int n, const Split& s, float inv,
                    const zero_step_control* ctl, double* ps, uint32_t* pf, hipStream_t stream) {
    const int64_t blocks = tile_blocks(s, kReduceTiles);
#define ZERO_REDUCE_CASE(K)                                                                    \
    case K:                                                                                    \
        return launch_pieces(s, blocks, [&](const Split& piece, int64_t g) {                   \
            return launch(reduce_kernel<DT, K, CHECK>, g, reduce_lds(K), stream, dst, src, piece, \
                          inv, ctl, ps, pf);                                                   \
        });
    switch (n) {
        ZERO_REDUCE_CASE(1) ZERO_REDUCE_CASE(2) ZERO_REDUCE_CASE(3) ZERO_REDUCE_CASE(4)
        ZERO_REDUCE_CASE(5) ZERO_REDUCE_CASE(6) ZERO_REDUCE_CASE(7) ZERO_REDUCE_CASE(8)
        ZERO_REDUCE_CASE(9) ZERO_REDUCE_CASE(10) ZERO_REDUCE_CASE(11) ZERO_REDUCE_CASE(12)
        ZERO_REDUCE_CASE(13) ZERO_REDUCE_CASE(14) ZERO_REDUCE_CASE(15) ZERO_REDUCE_CASE(16)
        default: return ZERO_EINVAL;
    }
#undef ZERO_REDUCE_CASE
}

// Checks shared by the reduce entry points; fills rank pointers and the split.
int reduce_args(void* dst, const void* const* srcs, int32_t n_ranks, int64_t count, int32_t dtype,
                RankPtrs* rp, Split* s) {
    if (count < 0 || n_ranks < 1 || n_ranks > ZERO_MAX_RANKS || !valid_dtype(dtype) || !srcs)
        return ZERO_EINVAL;
    const void* all16[ZERO_MAX_RANKS + 1];
    for (int r = 0; r < ZERO_MAX_RANKS; ++r) rp->p[r] = nullptr;
    for (int r = 0; r < n_ranks; ++r) {
        if (count > 0 && !srcs[r]) return ZERO_EINVAL;
        rp->p[r] = (const uint16_t*)srcs[r];
        all16[r] = srcs[r];
    }
    if (count > 0 && !dst) return ZERO_EINVAL;
    all16[n_ranks] = dst;
    *s = split_for(vector_head(all16, n_ranks + 1, nullptr, 0), count);
    return ZERO_OK;
}

int check_args(zero_step_result* res, void* workspace, size_t workspace_bytes, int64_t count,
               float inv_scale) {
    if (!res || !workspace || ((uintptr_t)workspace & 7) != 0) return ZERO_EINVAL;
    if (!(inv_scale > 0.0f) || !__builtin_isfinite(inv_scale)) return ZERO_EINVAL;
    if (workspace_bytes < zero_check_workspace_bytes(count)) return ZERO_EINVAL;
    return ZERO_OK;
}

// Check and fused reduce+check; the unscale factor is inv_scale, or read on
// the device from ctl when ctl is not null.
int check_impl(const void* grad16, int64_t count, int32_t dtype, float inv_scale,
               const zero_step_control* ctl, zero_step_result* res, void* workspace,
               size_t workspace_bytes, int32_t accumulate, hipStream_t stream) {
    if (count < 0 || !valid_dtype(dtype)) return ZERO_EINVAL;
    if (count > 0 && !grad16) return ZERO_EINVAL;
    int rc = check_args(res, workspace, workspace_bytes, count, inv_scale);
    if (rc != ZERO_OK) return rc;
    const void* p = grad16;
    const Split s = split_for(vector_head(&p, 1, nullptr, 0), count);
    const int64_t blocks = tile_blocks(s);
    const Levels L = levels_for(blocks);
    char* ws = (char*)workspace;
    double* ps = (double*)(ws + L.sum_off[0]);
    uint32_t* pf = (uint32_t*)(ws + L.flag_off[0]);
    const uint16_t* g = (const uint16_t*)grad16;
    rc = launch_pieces(s, blocks, [&](const Split& piece, int64_t grid) {
        return dtype == ZERO_FP16
                   ? launch(check_kernel<ZERO_FP16>, grid, 0, stream, g, piece, inv_scale, ctl,
                            ps, pf)
                   : launch(check_kernel<ZERO_BF16>, grid, 0, stream, g, piece, inv_scale, ctl,
                            ps, pf);
    });
    if (rc != ZERO_OK) return rc;
    return fold_into(ws, L, inv_scale, ctl, accumulate, res, stream);
}

int reduce_check_impl(void* dst, const void* const* srcs, int32_t n_ranks, int64_t count,
                      int32_t dtype, float inv_scale, const zero_step_control* ctl,
                      zero_step_result* res, void* workspace, size_t workspace_bytes,
                      int32_t accumulate, hipStream_t stream) {
    RankPtrs rp;
    Split s;
    int rc = reduce_args(dst, srcs, n_ranks, count, dtype, &rp, &s);
    if (rc != ZERO_OK) return rc;
    rc = check_args(res, workspace, workspace_bytes, count, inv_scale);
    if (rc != ZERO_OK) return rc;
    const int64_t blocks = tile_blocks(s, kReduceTiles);
    const Levels L = levels_for(blocks);
    char* ws = (char*)workspace;
    double* ps = (double*)(ws + L.sum_off[0]);
    uint32_t* pf = (uint32_t*)(ws + L.flag_off[0]);
    uint16_t* d = (uint16_t*)dst;
    rc = dtype == ZERO_FP16
             ? launch_reduce_n<ZERO_FP16, true>(d, rp, n_ranks, s, inv_scale, ctl, ps, pf, stream)
             : launch_reduce_n<ZERO_BF16, true>(d, rp, n_ranks, s, inv_scale, ctl, ps, pf, stream);
    if (rc != ZERO_OK) return rc;
    return fold_into(ws, L, inv_scale, ctl, accumulate, res, stream);
}

// The step's fp32 constants from hp, each rounded once from fp64; with
// device step control the betas and bias corrections come from ctl instead
// (read on the device).
AdamConsts adam_consts(const zero_adamw_hparams* hp, bool ctl) {
    AdamConsts c;
    const double t = ctl ? 1.0 : (double)hp->step;
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
    return c;
}

// 2 resident blocks per CU: 6.10 -> 6.37 TB/s on the LLaMA-70B-shaped shard,
// 5.33 -> 5.84 TB/s on the 7B one (MI355X).  Launches of at most
// kAdamSmallCount elements (the ToyModel and BERT-base owner shards) run 3
// per CU: 0.059 against 0.064 ms at 1.26e7 elements, while from 2.5e7
// elements on 2 per CU is faster.
constexpr int kAdamBlocksPerCU = 2;
constexpr int kAdamSmallBlocksPerCU = 3;
constexpr int64_t kAdamSmallCount = int64_t(1) << 24;
static_assert((kThreads / 64) * kAdamWaveBytes <= kLdsPerCU / (kAdamSmallBlocksPerCU + 1) + 2048u,
              "the AdamW caps' dynamic LDS holds every wave's staging area");

template <int DT>
int launch_adamw(float* master, float* exp_avg, float* exp_avg_sq, uint16_t* p16,
                 const uint16_t* g16, const Split& s, const AdamConsts& c,
                 const zero_step_control* ctl, const zero_step_result* res, hipStream_t stream) {
    const unsigned lds = lds_for_blocks(s.count <= kAdamSmallCount ? kAdamSmallBlocksPerCU
                                                                    : kAdamBlocksPerCU);
    return launch_pieces(s, tile_blocks(s), [&](const Split& piece, int64_t grid) {
        return launch(adamw_kernel<DT>, grid, lds, stream, master, exp_avg, exp_avg_sq, p16, g16,
                      piece, c, ctl, res);
    });
}

// AdamW over one partition; the step's betas and bias corrections come from
// hp (hp->step) or, when ctl is not null, from ctl on the device.
int adamw_impl(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
               const void* grad16, int64_t count, int32_t dtype, const zero_adamw_hparams* hp,
               const zero_step_control* ctl, const zero_step_result* res, hipStream_t stream) {
    if (count < 0 || !valid_dtype(dtype) || !res) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !param16 || !grad16) return ZERO_EINVAL;
    const AdamConsts c = adam_consts(hp, ctl != nullptr);
    const void* p16s[2] = {param16, grad16};
    const void* p32s[3] = {master, exp_avg, exp_avg_sq};
    const Split s = split_for(vector_head(p16s, 2, p32s, 3), count);
    uint16_t* p16 = (uint16_t*)param16;
    const uint16_t* g16 = (const uint16_t*)grad16;
    return dtype == ZERO_FP16
               ? launch_adamw<ZERO_FP16>(master, exp_avg, exp_avg_sq, p16, g16, s, c, ctl, res, stream)
               : launch_adamw<ZERO_BF16>(master, exp_avg, exp_avg_sq, p16, g16, s, c, ctl, res, stream);
}

// ------------------------------------------------------------- ranges -----
// A list of element ranges: offsets and counts >= 0, offset + count without
// int64 overflow, and no element in two ranges (empty ranges may sit
// anywhere).
int check_ranges(const zero_range* ranges, int32_t n, bool* any_elements) {
    *any_elements = false;
    if (n < 0 || (n > 0 && !ranges)) return ZERO_EINVAL;
    std::vector<std::pair<int64_t, int64_t>> v;
    v.reserve((size_t)n);
    for (int32_t r = 0; r < n; ++r) {
        const int64_t a = ranges[r].offset, c = ranges[r].count;
        if (a < 0 || c < 0) return ZERO_EINVAL;
        int64_t end;
        if (__builtin_add_overflow(a, c, &end)) return ZERO_ERANGE;
        if (c > 0) v.emplace_back(a, end);
    }
    std::sort(v.begin(), v.end());
    for (size_t k = 1; k < v.size(); ++k)
        if (v[k].first < v[k - 1].second) return ZERO_EINVAL;
    *any_elements = !v.empty();
    return ZERO_OK;
}

// The non-empty ranges of a checked list in offset order, with ranges that
// touch (one ends where the next begins) merged into one: every element is
// still updated once, each kernel's per-element work is independent, and one
// launch over the union avoids a launch tail and ramp per range (bucket
// group on MI355X: reduce 6.67 -> 6.37 ms, AdamW 5.30 -> 5.22 ms over 18 / 16
// touching ranges).
std::vector<zero_range> merged_ranges(const zero_range* ranges, int32_t n) {
    std::vector<zero_range> v;
    for (int32_t r = 0; r < n; ++r)
        if (ranges[r].count > 0) v.push_back(ranges[r]);
    std::sort(v.begin(), v.end(),
              [](const zero_range& x, const zero_range& y) { return x.offset < y.offset; });
    std::vector<zero_range> out;
    for (const zero_range& r : v) {
        if (!out.empty() && out.back().offset + out.back().count == r.offset)
            out.back().count += r.count;
        else
            out.push_back(r);
    }
    return out;
}

int64_t ranges_max_blocks(const zero_range* ranges, int32_t n) {
    int64_t b = 0;
    for (int32_t r = 0; r < n; ++r) b += max_tile_blocks(ranges[r].count > 0 ? ranges[r].count : 0);
    return b;
}

// Reduce+check over a list of ranges: each range is one launch of the
// single-range kernel (in pieces past one grid's size) reading its ranks at
// rp[r], its block partials written after the previous ranges' (range r's
// first partial at the sum of the earlier ranges' block counts), so the norm
// of all ranges is folded once.  (Packing several ranges into one launch
// made every block look up its range before its first load; the dependent
// scalar loads cost 2-4 %.)
template <int DT>
int reduce_check_ranges_t(uint16_t* dst, const std::vector<RankPtrs>& rp, int32_t n_ranks,
                          const zero_range* ranges, int32_t n, float inv,
                          const zero_step_control* ctl, double* ps, uint32_t* pf,
                          const std::vector<Split>& splits, const std::vector<int64_t>& blocks,
                          hipStream_t stream) {
    int64_t base = 0;
    for (int32_t r = 0; r < n; ++r) {
        const int rc = launch_reduce_n<DT, true>(dst + ranges[r].offset, rp[r], n_ranks, splits[r],
                                                 inv, ctl, ps + base, pf + base, stream);
        if (rc != ZERO_OK) return rc;
        base += blocks[r];
    }
    return ZERO_OK;
}

// Checks of the arguments the range-list reduce calls share.
int reduce_list_args(int32_t n_ranks, int32_t dtype, const void* srcs, float inv_scale,
                     const zero_step_result* res, const void* workspace) {
    if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS || !valid_dtype(dtype) || !srcs) return ZERO_EINVAL;
    if (!res || !workspace || ((uintptr_t)workspace & 7) != 0) return ZERO_EINVAL;
    if (!(inv_scale > 0.0f) || !__builtin_isfinite(inv_scale)) return ZERO_EINVAL;
    return ZERO_OK;
}

// Launches the ranges (each with its own rank pointers) and folds the norm.
int reduce_check_list(uint16_t* d, const std::vector<RankPtrs>& rps,
                      const std::vector<zero_range>& rs, int32_t n_ranks, int32_t dtype,
                      float inv_scale, const zero_step_control* ctl, zero_step_result* res,
                      void* workspace, int32_t accumulate, hipStream_t stream) {
    std::vector<Split> splits;
    std::vector<int64_t> blocks;
    int64_t total = 0;
    for (size_t w = 0; w < rs.size(); ++w) {
        const void* all16[ZERO_MAX_RANKS + 1];
        for (int k = 0; k < n_ranks; ++k) all16[k] = rps[w].p[k];
        all16[n_ranks] = d + rs[w].offset;
        splits.push_back(split_for(vector_head(all16, n_ranks + 1, nullptr, 0), rs[w].count));
        blocks.push_back(tile_blocks(splits.back(), kReduceTiles));
        total += blocks.back();
    }
    const int32_t m = (int32_t)rs.size();
    const Levels L = levels_for(total);
    char* ws = (char*)workspace;
    double* ps = (double*)(ws + L.sum_off[0]);
    uint32_t* pf = (uint32_t*)(ws + L.flag_off[0]);
    const int rc = dtype == ZERO_FP16
                       ? reduce_check_ranges_t<ZERO_FP16>(d, rps, n_ranks, rs.data(), m, inv_scale,
                                                          ctl, ps, pf, splits, blocks, stream)
                       : reduce_check_ranges_t<ZERO_BF16>(d, rps, n_ranks, rs.data(), m, inv_scale,
                                                          ctl, ps, pf, splits, blocks, stream);
    if (rc != ZERO_OK) return rc;
    return fold_into(ws, L, inv_scale, ctl, accumulate, res, stream);
}

int reduce_check_ranges_impl(void* dst, const void* const* srcs, int32_t n_ranks,
                             const zero_range* ranges, int32_t n, int32_t dtype, float inv_scale,
                             const zero_step_control* ctl, zero_step_result* res, void* workspace,
                             size_t workspace_bytes, int32_t accumulate, hipStream_t stream) {
    int rc = reduce_list_args(n_ranks, dtype, srcs, inv_scale, res, workspace);
    if (rc != ZERO_OK) return rc;
    bool any = false;
    rc = check_ranges(ranges, n, &any);
    if (rc != ZERO_OK) return rc;
    if (any && !dst) return ZERO_EINVAL;
    RankPtrs rp;
    for (int r = 0; r < ZERO_MAX_RANKS; ++r) rp.p[r] = nullptr;
    for (int r = 0; r < n_ranks; ++r) {
        if (any && !srcs[r]) return ZERO_EINVAL;
        rp.p[r] = (const uint16_t*)srcs[r];
    }
    if (workspace_bytes < levels_for(ranges_max_blocks(ranges, n)).bytes) return ZERO_EINVAL;
    // empty ranges take no blocks and touching ones are merged (with no
    // elements at all only the result is written, or left as it is when
    // accumulating); the workspace bound above holds for the merged list
    const std::vector<zero_range> rs = merged_ranges(ranges, n);
    std::vector<RankPtrs> rps;
    for (const zero_range& rg : rs) {
        RankPtrs sr = rp;
        for (int k = 0; k < n_ranks; ++k) sr.p[k] = rp.p[k] + rg.offset;
        rps.push_back(sr);
    }
    return reduce_check_list((uint16_t*)dst, rps, rs, n_ranks, dtype, inv_scale, ctl, res,
                             workspace, accumulate, stream);
}

int reduce_check_buckets_impl(void* dst, const void* const* srcs, int32_t n_ranks,
                              const zero_range* windows, int32_t n, int32_t dtype,
                              float inv_scale, const zero_step_control* ctl,
                              zero_step_result* res, void* workspace, size_t workspace_bytes,
                              int32_t accumulate, hipStream_t stream) {
    int rc = reduce_list_args(n_ranks, dtype, srcs, inv_scale, res, workspace);
    if (rc != ZERO_OK) return rc;
    bool any = false;
    rc = check_ranges(windows, n, &any);
    if (rc != ZERO_OK) return rc;
    if (any && !dst) return ZERO_EINVAL;
    if (workspace_bytes < levels_for(ranges_max_blocks(windows, n)).bytes) return ZERO_EINVAL;
    // every non-empty window in list order, each with its own rank buffers
    std::vector<zero_range> rs;
    std::vector<RankPtrs> rps;
    for (int32_t w = 0; w < n; ++w) {
        if (windows[w].count == 0) continue;
        RankPtrs sr;
        for (int r = 0; r < ZERO_MAX_RANKS; ++r) sr.p[r] = nullptr;
        for (int r = 0; r < n_ranks; ++r) {
            const void* p = srcs[(size_t)w * n_ranks + r];
            if (!p) return ZERO_EINVAL;
            sr.p[r] = (const uint16_t*)p;
        }
        rs.push_back(windows[w]);
        rps.push_back(sr);
    }
    return reduce_check_list((uint16_t*)dst, rps, rs, n_ranks, dtype, inv_scale, ctl, res,
                             workspace, accumulate, stream);
}

template <int DT>
int adamw_ranges_t(float* master, float* ma, float* va, uint16_t* p16, const uint16_t* g16,
                   const zero_range* ranges, int32_t n, const AdamConsts& c,
                   const zero_step_control* ctl, const zero_step_result* res,
                   const std::vector<Split>& splits, hipStream_t stream) {
    for (int32_t r = 0; r < n; ++r) {
        const int64_t off = ranges[r].offset;
        const int rc = launch_adamw<DT>(master + off, ma + off, va + off, p16 + off, g16 + off,
                                        splits[r], c, ctl, res, stream);
        if (rc != ZERO_OK) return rc;
    }
    return ZERO_OK;
}

int adamw_ranges_impl(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                      const void* grad16, const zero_range* ranges, int32_t n, int32_t dtype,
                      const zero_adamw_hparams* hp, const zero_step_control* ctl,
                      const zero_step_result* res, hipStream_t stream) {
    if (!valid_dtype(dtype) || !res || !hp) return ZERO_EINVAL;
    if (!ctl && hp->step < 1) return ZERO_EINVAL;
    bool any = false;
    const int rc = check_ranges(ranges, n, &any);
    if (rc != ZERO_OK) return rc;
    if (!any) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !param16 || !grad16) return ZERO_EINVAL;
    const AdamConsts c = adam_consts(hp, ctl != nullptr);
    uint16_t* p16 = (uint16_t*)param16;
    const uint16_t* g16 = (const uint16_t*)grad16;
    // empty ranges take no blocks and touching ones are merged
    const std::vector<zero_range> rs = merged_ranges(ranges, n);
    std::vector<Split> splits;
    for (const zero_range& rg : rs) {
        const int64_t off = rg.offset;
        const void* p16s[2] = {p16 + off, g16 + off};
        const void* p32s[3] = {master + off, exp_avg + off, exp_avg_sq + off};
        splits.push_back(split_for(vector_head(p16s, 2, p32s, 3), rg.count));
    }
    const int32_t m = (int32_t)rs.size();
    return dtype == ZERO_FP16
               ? adamw_ranges_t<ZERO_FP16>(master, exp_avg, exp_avg_sq, p16, g16, rs.data(), m, c,
                                           ctl, res, splits, stream)
               : adamw_ranges_t<ZERO_BF16>(master, exp_avg, exp_avg_sq, p16, g16, rs.data(), m, c,
                                           ctl, res, splits, stream);
}

}  // namespace

// ------------------------------------------------ allocation-free variant --
// zero_reduce_check_owned_noalloc keeps the check partials (the workspace of
// the other calls) in `scratch`, one copy per device for the life of the
// process, so that callers that cannot allocate need no workspace.  It takes
// up to kNoAllocMaxCount elements; kScratchBytes is the workspace that count
// needs (24 MiB).
namespace {
constexpr int64_t kNoAllocMaxCount = int64_t(1) << 32;

constexpr size_t workspace_bound(int64_t blocks) {
    size_t off = 0;
    int64_t n = blocks;
    while (true) {
        off += (size_t)n * sizeof(double);
        off += ((size_t)n * sizeof(uint32_t) + 7) & ~(size_t)7;
        if (n <= kFinal) break;
        n = (n + kFold - 1) / kFold;
    }
    return off;
}
constexpr size_t kScratchBytes =
    (workspace_bound((kNoAllocMaxCount + kTile - 1) / kTile + 1) + 255) / 256 * 256;
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device

// The device address of `scratch` on the device that runs `stream` (the
// current device for the null stream), looked up once per device with that
// device current.
int scratch_for_stream(hipStream_t stream, void** out) {
    int dev = 0;
    if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return ZERO_EDEVICE;
    if (dev < 0 || dev >= kMaxDevices) return ZERO_EDEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return ZERO_EDEVICE;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return ZERO_EDEVICE;
        void* p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return ZERO_EDEVICE;
        if (err != hipSuccess || !p) return ZERO_EDEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ZERO_OK;
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
    const unsigned grid = stream_grid(count);
    const uint16_t* p = (const uint16_t*)param16;
    return dtype == ZERO_FP16
               ? launch(init_master_kernel<ZERO_FP16>, grid, 0, stream, master, p, count)
               : launch(init_master_kernel<ZERO_BF16>, grid, 0, stream, master, p, count);
}

int zero_reduce_owned(void* dst, const void* const* srcs, int32_t n_ranks, int64_t count,
                      int32_t dtype, hipStream_t stream) {
    RankPtrs rp;
    Split s;
    int rc = reduce_args(dst, srcs, n_ranks, count, dtype, &rp, &s);
    if (rc != ZERO_OK || count == 0) return rc;
    uint16_t* d = (uint16_t*)dst;
    return dtype == ZERO_FP16
               ? launch_reduce_n<ZERO_FP16, false>(d, rp, n_ranks, s, 0.0f, nullptr, nullptr,
                                                   nullptr, stream)
               : launch_reduce_n<ZERO_BF16, false>(d, rp, n_ranks, s, 0.0f, nullptr, nullptr,
                                                   nullptr, stream);
}

size_t zero_check_workspace_bytes(int64_t count) {
    if (count < 0) count = 0;
    return levels_for(max_tile_blocks(count)).bytes;
}

int zero_unscale_check_norm(const void* grad16, int64_t count, int32_t dtype, float inv_scale,
                            zero_step_result* res, void* workspace, size_t workspace_bytes,
                            int32_t accumulate, hipStream_t stream) {
    return check_impl(grad16, count, dtype, inv_scale, nullptr, res, workspace, workspace_bytes,
                      accumulate, stream);
}

int zero_unscale_check_norm_ctl(const void* grad16, int64_t count, int32_t dtype,
                                const zero_step_control* ctl, zero_step_result* res,
                                void* workspace, size_t workspace_bytes, int32_t accumulate,
                                hipStream_t stream) {
    if (!ctl) return ZERO_EINVAL;
    return check_impl(grad16, count, dtype, 1.0f, ctl, res, workspace, workspace_bytes,
                      accumulate, stream);
}

int zero_reduce_check_owned(void* dst, const void* const* srcs, int32_t n_ranks, int64_t count,
                            int32_t dtype, float inv_scale, zero_step_result* res, void* workspace,
                            size_t workspace_bytes, int32_t accumulate, hipStream_t stream) {
    return reduce_check_impl(dst, srcs, n_ranks, count, dtype, inv_scale, nullptr, res, workspace,
                             workspace_bytes, accumulate, stream);
}

int zero_reduce_check_owned_noalloc(void* dst, const void* const* srcs, int32_t n_ranks,
                                    int64_t count, int32_t dtype, float inv_scale,
                                    zero_step_result* res, int32_t accumulate,
                                    hipStream_t stream) {
    if (count < 0) return ZERO_EINVAL;
    if (count > kNoAllocMaxCount) return ZERO_ERANGE;
    void* ws = nullptr;
    const int rc = scratch_for_stream(stream, &ws);
    if (rc != ZERO_OK) return rc;
    return reduce_check_impl(dst, srcs, n_ranks, count, dtype, inv_scale, nullptr, res, ws,
                             kScratchBytes, accumulate, stream);
}

int zero_reduce_check_owned_ctl(void* dst, const void* const* srcs, int32_t n_ranks,
                                int64_t count, int32_t dtype, const zero_step_control* ctl,
                                zero_step_result* res, void* workspace, size_t workspace_bytes,
                                int32_t accumulate, hipStream_t stream) {
    if (!ctl) return ZERO_EINVAL;
    return reduce_check_impl(dst, srcs, n_ranks, count, dtype, 1.0f, ctl, res, workspace,
                             workspace_bytes, accumulate, stream);
}

int zero_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                    const void* grad16, int64_t count, int32_t dtype,
                    const zero_adamw_hparams* hp, const zero_step_result* res,
                    hipStream_t stream) {
    if (!hp || hp->step < 1) return ZERO_EINVAL;
    return adamw_impl(master, exp_avg, exp_avg_sq, param16, grad16, count, dtype, hp, nullptr, res,
                      stream);
}

int zero_adamw_step_ctl(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                        const void* grad16, int64_t count, int32_t dtype,
                        const zero_adamw_hparams* hp, const zero_step_control* ctl,
                        const zero_step_result* res, hipStream_t stream) {
    if (!hp || !ctl) return ZERO_EINVAL;
    return adamw_impl(master, exp_avg, exp_avg_sq, param16, grad16, count, dtype, hp, ctl, res,
                      stream);
}

size_t zero_range_workspace_bytes(const zero_range* ranges, int32_t n_ranges) {
    bool any = false;
    if (check_ranges(ranges, n_ranges, &any) != ZERO_OK) return 0;
    return levels_for(ranges_max_blocks(ranges, n_ranges)).bytes;
}

int zero_reduce_check_ranges(void* dst, const void* const* srcs, int32_t n_ranks,
                             const zero_range* ranges, int32_t n_ranges, int32_t dtype,
                             float inv_scale, const zero_step_control* ctl,
                             zero_step_result* res, void* workspace, size_t workspace_bytes,
                             int32_t accumulate, hipStream_t stream) {
    return reduce_check_ranges_impl(dst, srcs, n_ranks, ranges, n_ranges, dtype,
                                    ctl ? 1.0f : inv_scale, ctl, res, workspace, workspace_bytes,
                                    accumulate, stream);
}

int zero_reduce_check_buckets(void* dst, const void* const* srcs, int32_t n_ranks,
                              const zero_range* windows, int32_t n_windows, int32_t dtype,
                              float inv_scale, const zero_step_control* ctl,
                              zero_step_result* res, void* workspace, size_t workspace_bytes,
                              int32_t accumulate, hipStream_t stream) {
    return reduce_check_buckets_impl(dst, srcs, n_ranks, windows, n_windows, dtype,
                                     ctl ? 1.0f : inv_scale, ctl, res, workspace, workspace_bytes,
                                     accumulate, stream);
}

int zero_adamw_step_ranges(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                           const void* grad16, const zero_range* ranges, int32_t n_ranges,
                           int32_t dtype, const zero_adamw_hparams* hp,
                           const zero_step_control* ctl, const zero_step_result* res,
                           hipStream_t stream) {
    return adamw_ranges_impl(master, exp_avg, exp_avg_sq, param16, grad16, ranges, n_ranges,
                             dtype, hp, ctl, res, stream);
}

int zero_step_control_init(zero_step_control* ctl, double scale0, double min_scale,
                           int64_t window, float divisor, float beta1, float beta2) {
    if (!ctl || !(scale0 > 0.0) || !__builtin_isfinite(scale0) || !(min_scale > 0.0) ||
        !__builtin_isfinite(min_scale) || window < 1 || !(divisor > 0.0f) ||
        !__builtin_isfinite(divisor) || !(beta1 >= 0.0f && beta1 < 1.0f) ||
        !(beta2 >= 0.0f && beta2 < 1.0f))
        return ZERO_EINVAL;
    zero_step_control c;
    c.scale = scale0;
    c.min_scale = min_scale;
    c.window = window;
    c.clean = 0;
    c.skipped = 0;
    c.t = 0;
    c.divisor = divisor;
    c.inv_scale = (float)(1.0 / (scale0 * (double)divisor));
    c.beta1 = beta1;
    c.beta2 = beta2;
    c.bc1 = (float)(1.0 - pow((double)beta1, 1.0));
    c.bc2 = (float)(1.0 - pow((double)beta2, 1.0));
    *ctl = c;
    return ZERO_OK;
}

int zero_step_control_update(zero_step_control* ctl, const zero_step_result* res,
                             hipStream_t stream) {
    if (!ctl || !res) return ZERO_EINVAL;
    return launch_shape(control_update_kernel, 1, 64, 0u, stream, ctl, res);
}

}  // extern "C"
