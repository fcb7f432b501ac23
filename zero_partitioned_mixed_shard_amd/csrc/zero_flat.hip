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

// Gather: one 8-element tile of the flat buffer per lane (aligned through
// the head split); a tile inside one tensor takes the 128-bit path, others
// go element by element.  Thread 0 finds the block's first tensor by binary
// search; lanes walk forward from it.
__global__ void __launch_bounds__(kThreads)
flat_gather_kernel(uint16_t* __restrict__ flat, Split s, const zero_tensor_desc* __restrict__ descs,
                   int64_t n_descs) {
    __shared__ int64_t s_first;
    const int64_t blk = block_id(s);
    const int64_t base = s.aligned ? s.head + blk * kTile : blk * kTile;
    if (threadIdx.x == 0) s_first = desc_at(descs, n_descs, blk == 0 ? 0 : base);
    __syncthreads();
    DescCursor cur;
    cur.d = descs;
    cur.n = n_descs;
    cur.load(s_first);
    const int64_t i = lane_tile(s);
    const int64_t e0 = s.aligned ? s.head + i * kVec : i * kVec;
    const bool vec_lane = s.aligned && i < s.nvec;
    if (vec_lane || (!s.aligned && e0 < s.count)) {
        cur.seek(e0);
        const int64_t j0 = cur.index(e0);
        if (vec_lane && j0 >= 0 && j0 + kVec <= cur.numel) {
            store_nt(flat + e0, load8_unaligned(cur.ptr + j0));
        } else {
            for (int64_t e = e0; e < e0 + kVec && e < s.count; ++e) {
                cur.seek(e);
                const int64_t j = cur.index(e);
                flat[e] = j >= 0 ? cur.ptr[j] : (uint16_t)0;
            }
        }
    }
    if (s.aligned && blk == 0) {             // head and tail, one element per lane
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
            flat[e] = j >= 0 ? c2.ptr[j] : (uint16_t)0;
        }
    }
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

// Scatter: one 8-element tile of the flat buffer per lane (aligned through
// the head split), the mirror of the gather.
__global__ void __launch_bounds__(kThreads)
flat_scatter_kernel(const uint16_t* __restrict__ flat, Split s,
                    const zero_tensor_desc* __restrict__ descs, int64_t n_descs) {
    __shared__ int64_t s_first;
    const int64_t blk = block_id(s);
    const int64_t base = s.aligned ? s.head + blk * kTile : blk * kTile;
    if (threadIdx.x == 0) s_first = desc_at(descs, n_descs, blk == 0 ? 0 : base);
    __syncthreads();
    DescCursor cur;
    cur.d = descs;
    cur.n = n_descs;
    cur.load(s_first);
    const int64_t i = lane_tile(s);
    const int64_t e0 = s.aligned ? s.head + i * kVec : i * kVec;
    const bool vec_lane = s.aligned && i < s.nvec;
    if (vec_lane || (!s.aligned && e0 < s.count)) {
        cur.seek(e0);
        const int64_t j0 = cur.index(e0);
        if (vec_lane && j0 >= 0 && j0 + kVec <= cur.numel) {
            store8_unaligned(cur.ptr + j0, load_nt(flat + e0));
        } else {
            for (int64_t e = e0; e < e0 + kVec && e < s.count; ++e) {
                cur.seek(e);
                const int64_t j = cur.index(e);
                if (j >= 0) cur.ptr[j] = flat[e];
            }
        }
    }
    if (s.aligned && blk == 0) {             // head and tail, one element per lane
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
            if (j >= 0) c2.ptr[j] = flat[e];
        }
    }
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
    return launch_pieces(s, tile_blocks(s), [&](const Split& piece, int64_t grid) {
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
    return launch_pieces(s, tile_blocks(s), [&](const Split& piece, int64_t grid) {
        return launch(flat_scatter_kernel, grid, 0, stream, (const uint16_t*)flat, piece, descs,
                      n_descs);
    });
}

}  // extern "C"
