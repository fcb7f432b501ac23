// zero_flat.hip -- bucket copy-in and write-back between per-tensor 16-bit
// buffers and a flat buffer (zero_flat_gather / zero_flat_scatter, declared
// in include/zero_shard.h).  Tile geometry and launch as in zero_shard.hip.

#include "zero_common.h"

namespace {

// ------------------------------------------- flat <-> tensors (copy) -------
// Last descriptor whose offset is <= e, or -1.
__device__ __forceinline__ int64_t desc_at(const zero_tensor_desc* d, int64_t n, int64_t e) {
    int64_t lo = 0, hi = n;                  // first index with offset > e
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (d[mid].offset <= e) lo = mid + 1;
        else hi = mid;
    }
    return lo - 1;
}

// Index of the last descriptor whose offset is <= e, or -1, found by one
// whole wave: each round tests 64 evenly spaced descriptors at once and keeps
// the interval between the last one at or below e and the next, so a table
// of n entries costs ceil(log64 n) dependent loads (a binary search by one
// thread: log2 n; on a 3,300-tensor bucket 2 loads instead of 12, which
// matters because every block waits for it).  Every lane of the wave calls
// it with the same e.  Every index it reads lies in [0, n), whatever the
// table holds.
__device__ __forceinline__ int64_t wave_desc_at(const zero_tensor_desc* d, int64_t n, int64_t e) {
    const int lane = threadIdx.x & 63;
    int64_t lo = 0, hi = n;           // lo == 0 or d[lo].offset <= e; answer in [lo - 1, hi)
    while (hi - lo > 64) {
        const int64_t step = (hi - lo + 63) / 64;
        const int64_t j = lo + (int64_t)lane * step;
        const bool le = j < hi && d[j].offset <= e;
        const int c = __popcll(__ballot(le));
        if (c == 0) return lo - 1;    // only when lo == 0: e lies before every tensor
        const int64_t nhi = lo + (int64_t)c * step;
        lo = lo + (int64_t)(c - 1) * step;
        hi = nhi < hi ? nhi : hi;
    }
    const int64_t j = lo + lane;
    const bool le = j < hi && d[j].offset <= e;
    return lo + __popcll(__ballot(le)) - 1;
}

// A lane's view of the descriptor table: the tensor holding the flat
// elements it is at, advanced forward only.
struct DescCursor {
    const zero_tensor_desc* d;
    int64_t n, k, off, numel, next;
    uint16_t* ptr;

    __device__ __forceinline__ void load(int64_t kk) {
        k = kk;
        ptr = nullptr;
        off = 0;
        numel = 0;
        if (k >= 0) {
            ptr = (uint16_t*)d[k].ptr;
            off = d[k].offset;
            numel = d[k].numel;
        }
        next = k + 1 < n ? d[k + 1].offset : INT64_MAX;
    }
    __device__ __forceinline__ void seek(int64_t e) {   // e never decreases
        while (next <= e) load(k + 1);
    }
    // index of flat element e in the current tensor, or -1 if e is in a gap
    __device__ __forceinline__ int64_t index(int64_t e) const {
        const int64_t j = e - off;
        return (k >= 0 && j >= 0 && j < numel) ? j : -1;
    }
};

// 8 consecutive 16-bit values starting at a 2-byte aligned address, read as
// the two aligned 16-byte chunks that hold them.  Both chunks lie in the
// pages of the first and last value, so nothing outside them is touched.
__device__ __forceinline__ u32x4 load8_unaligned(const uint16_t* p) {
    const uintptr_t a = (uintptr_t)p;
    const u32x4* c = (const u32x4*)(a & ~(uintptr_t)15);
    const int sh = (int)((a & 15) >> 1);     // 0..7 elements into the first chunk
    const u32x4 c0 = __builtin_nontemporal_load(c);
    if (sh == 0) return c0;
    const u32x4 c1 = __builtin_nontemporal_load(c + 1);
    const uint32_t w[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    u32x4 o;
    switch (sh) {
#define ZERO_EVEN(T) case 2 * T: o[0] = w[T]; o[1] = w[T + 1]; o[2] = w[T + 2]; o[3] = w[T + 3]; break;
#define ZERO_ODD(T)                                            \
    case 2 * T + 1:                                            \
        o[0] = __builtin_amdgcn_alignbit(w[T + 1], w[T], 16);  \
        o[1] = __builtin_amdgcn_alignbit(w[T + 2], w[T + 1], 16); \
        o[2] = __builtin_amdgcn_alignbit(w[T + 3], w[T + 2], 16); \
        o[3] = __builtin_amdgcn_alignbit(w[T + 4], w[T + 3], 16); \
        break;
        ZERO_ODD(0) ZERO_EVEN(1) ZERO_ODD(1) ZERO_EVEN(2) ZERO_ODD(2) ZERO_EVEN(3) ZERO_ODD(3)
#undef ZERO_EVEN
#undef ZERO_ODD
        default: o = c0; break;
    }
    return o;
}

// 8 consecutive 16-bit values (packed in w) to a 2-byte aligned address:
// one 16-byte store when the address is 4-byte aligned, else a 16-bit store,
// a 12-byte store and a 16-bit store.  Only these 16 bytes are written.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));

__device__ __forceinline__ void store8_unaligned(uint16_t* p, u32x4 w) {
    if (((uintptr_t)p & 3) == 0) {
        *reinterpret_cast<u32x4_a4*>(p) = w;
        return;
    }
    p[0] = (uint16_t)(w[0] & 0xFFFFu);
    u32x3_a4 mid;
    mid[0] = __builtin_amdgcn_alignbit(w[1], w[0], 16);
    mid[1] = __builtin_amdgcn_alignbit(w[2], w[1], 16);
    mid[2] = __builtin_amdgcn_alignbit(w[3], w[2], 16);
    *reinterpret_cast<u32x3_a4*>(p + 1) = mid;
    p[7] = (uint16_t)(w[3] >> 16);
}

// Block-wide rows of lane tiles per block in the copy kernels: the block's
// dependent lookups (the descriptor search, the first descriptor) are paid
// once for 4 rows, and a lane has the loads of all 4 rows in flight at once.
constexpr int kFlatRows = 4;

// First descriptor at or below flat element e for the whole block (wave 0
// searches, LDS broadcasts).  Every thread of the block calls it.
__device__ __forceinline__ int64_t block_first_desc(const zero_tensor_desc* d, int64_t n, int64_t e) {
    __shared__ int64_t s_first;
    if (threadIdx.x < 64) {
        const int64_t k = wave_desc_at(d, n, e);
        if (threadIdx.x == 0) s_first = k;
    }
    __syncthreads();
    return s_first;
}

// Copy between the flat buffer and the tensors the descriptors name
// (GATHER: tensors -> flat, zero where no tensor; else flat -> tensors).
// A lane owns one 8-element tile in each of the block's kFlatRows rows
// (aligned through the head split); a tile inside one tensor takes the
// 128-bit path, others go element by element.  The lane walks the
// descriptor table forward from the block's first tensor, issues the loads
// of every row, then the stores.  Block 0 also does the head and tail
// elements one per lane.  `flat` is only read when !GATHER.
template <bool GATHER>
__device__ __forceinline__ void flat_copy(uint16_t* flat, const Split& s,
                                          const zero_tensor_desc* descs, int64_t n_descs) {
    const int64_t blk = block_id(s);
    const int64_t base = (s.aligned ? s.head : 0) + blk * (int64_t)kTile * kFlatRows;
    DescCursor cur;
    cur.d = descs;
    cur.n = n_descs;
    cur.load(block_first_desc(descs, n_descs, blk == 0 ? 0 : base));
    u32x4 v[kFlatRows];
    uint16_t* to[kFlatRows];
    bool fast[kFlatRows];
#pragma unroll
    for (int t = 0; t < kFlatRows; ++t) {
        fast[t] = false;
        const int64_t i = lane_tile<kFlatRows>(s, t);
        const int64_t e0 = s.aligned ? s.head + i * kVec : i * kVec;
        const bool vec_lane = s.aligned && i < s.nvec;
        if (!vec_lane && (s.aligned || e0 >= s.count)) continue;
        cur.seek(e0);
        const int64_t j0 = cur.index(e0);
        if (vec_lane && j0 >= 0 && j0 + kVec <= cur.numel) {
            if (GATHER) {
                v[t] = load8_unaligned(cur.ptr + j0);
                to[t] = flat + e0;
            } else {
                v[t] = load_nt(flat + e0);
                to[t] = cur.ptr + j0;
            }
            fast[t] = true;
        } else {
            for (int64_t e = e0; e < e0 + kVec && e < s.count; ++e) {
                cur.seek(e);
                const int64_t j = cur.index(e);
                if (GATHER) flat[e] = j >= 0 ? cur.ptr[j] : (uint16_t)0;
                else if (j >= 0) cur.ptr[j] = flat[e];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kFlatRows; ++t) {
        if (!fast[t]) continue;
        if (GATHER) store_nt(to[t], v[t]);
        else store8_unaligned(to[t], v[t]);
    }
    if (s.aligned && blk == 0) {
        const int t = threadIdx.x;
        int64_t e = -1;
        if (t < s.head) e = t;
        else if (t >= 64 && t < 64 + kVec && s.head + s.nvec * kVec + (t - 64) < s.count)
            e = s.head + s.nvec * kVec + (t - 64);
        if (e >= 0) {
            DescCursor c2;
            c2.d = descs;
            c2.n = n_descs;
            c2.load(desc_at(descs, n_descs, e));
            const int64_t j = c2.index(e);
            if (GATHER) flat[e] = j >= 0 ? c2.ptr[j] : (uint16_t)0;
            else if (j >= 0) c2.ptr[j] = flat[e];
        }
    }
}

__global__ void __launch_bounds__(kThreads)
flat_gather_kernel(uint16_t* flat, Split s, const zero_tensor_desc* __restrict__ descs,
                   int64_t n_descs) {
    flat_copy<true>(flat, s, descs, n_descs);
}

__global__ void __launch_bounds__(kThreads)
flat_scatter_kernel(const uint16_t* flat, Split s, const zero_tensor_desc* __restrict__ descs,
                    int64_t n_descs) {
    flat_copy<false>(const_cast<uint16_t*>(flat), s, descs, n_descs);
}

}  // namespace

extern "C" {

int zero_flat_gather(void* flat, int64_t flat_count, const zero_tensor_desc* descs,
                     int64_t n_descs, hipStream_t stream) {
    if (flat_count < 0 || n_descs < 0) return ZERO_EINVAL;
    if (flat_count == 0) return ZERO_OK;
    if (!flat || (n_descs > 0 && !descs)) return ZERO_EINVAL;
    const void* p = flat;
    const Split s = split_for(vector_head(&p, 1, nullptr, 0), flat_count);
    return launch_pieces(s, tile_blocks(s, kFlatRows), [&](const Split& piece, int64_t grid) {
        return launch(flat_gather_kernel, grid, 0, stream, (uint16_t*)flat, piece, descs, n_descs);
    });
}

int zero_flat_scatter(const void* flat, int64_t flat_count, const zero_tensor_desc* descs,
                      int64_t n_descs, hipStream_t stream) {
    if (flat_count < 0 || n_descs < 0) return ZERO_EINVAL;
    if (flat_count == 0 || n_descs == 0) return ZERO_OK;
    if (!flat || !descs) return ZERO_EINVAL;
    const void* p = flat;
    const Split s = split_for(vector_head(&p, 1, nullptr, 0), flat_count);
    return launch_pieces(s, tile_blocks(s, kFlatRows), [&](const Split& piece, int64_t grid) {
        return launch(flat_scatter_kernel, grid, 0, stream, (const uint16_t*)flat, piece, descs,
                      n_descs);
    });
}

}  // extern "C"
