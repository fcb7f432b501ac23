// zero_flat.hip -- bucket copy-in and write-back between per-tensor 16-bit
// buffers and a flat buffer (zero_flat_gather / zero_flat_scatter, declared
// in include/zero_shard.h).  Tile geometry and launch as in zero_shard.hip.

#include "zero_common.h"

namespace {

// Tensor pointers are read from the descriptor table, so the compiler cannot
// tell that they point to global memory and would emit flat (generic)
// accesses, whose completion is counted together with LDS and cross-lane
// operations; these types make them global accesses.
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) const u32x4 g_cu32x4;
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) uint64_t g_u64;

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
    g_u16* ptr;

    __device__ __forceinline__ void load(int64_t kk) {
        k = kk;
        ptr = nullptr;
        off = 0;
        numel = 0;
        if (k >= 0) {
            ptr = (g_u16*)d[k].ptr;
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

// The 8 16-bit values starting at element sh (0..7) of the 16 held in the
// aligned chunks c0, c1 (c0 first).
__device__ __forceinline__ u32x4 window8(u32x4 c0, u32x4 c1, int sh) {
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

// The next lane's copy of x (lane 63 gets 0): a DPP wave shift, which moves
// data between lanes in the VALU without the LDS crossbar.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x130 /* wave_shl:1 */, 0xF, 0xF,
                                                 false);
}

// Stores elements [first, first + n) (n <= 7) of the 8 packed in w to
// p[0, n) with at most four naturally aligned stores (2, 4 and 8 bytes).
__device__ __forceinline__ void store_elems(g_u16* p, u32x4 w, int first, int n) {
    const u32x4 zero = {0, 0, 0, 0};
    u32x4 u = window8(w, zero, first);     // element `first` first
    if (n > 0 && ((uintptr_t)p & 2)) {
        *p = (uint16_t)(u[0] & 0xFFFFu);
        u = window8(u, zero, 1);
        p += 1;
        n -= 1;
    }
    if (n >= 2 && ((uintptr_t)p & 4)) {
        *(g_u32*)p = u[0];
        u = u32x4{u[1], u[2], u[3], 0};
        p += 2;
        n -= 2;
    }
    if (n >= 4) {
        *(g_u64*)p = (uint64_t)u[0] | ((uint64_t)u[1] << 32);
        u = u32x4{u[2], u[3], 0, 0};
        p += 4;
        n -= 4;
    }
    if (n >= 2) {
        *(g_u32*)p = u[0];
        u = u32x4{u[1], u[2], u[3], 0};
        p += 2;
        n -= 2;
    }
    if (n >= 1) *p = (uint16_t)(u[0] & 0xFFFFu);
}

// Block-wide rows of lane tiles per block in the copy kernels: the block's
// dependent lookups (the descriptor search, the first descriptor) are paid
// once for 4 rows, and a lane has the loads of all 4 rows in flight at once.
constexpr int kFlatRows = 4;

// The block's cursor at flat element e: the last descriptor at or below e
// and the next one's offset, found by wave 0 with a 64-wide search (each
// round tests 64 evenly spaced descriptors at once) and broadcast through
// LDS.  Every thread of the block calls it; every index it reads lies in
// [0, n), whatever the table holds.
__device__ __forceinline__ void block_first_cursor(DescCursor& cur, const zero_tensor_desc* d,
                                                   int64_t n, int64_t e) {
    __shared__ int64_t s_k, s_off, s_numel, s_next;
    __shared__ g_u16* s_ptr;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int64_t lo = 0, hi = n;           // lo == 0 or d[lo].offset <= e; answer in [lo - 1, hi)
        int64_t k = -2;
        while (hi - lo > 63) {
            const int64_t step = (hi - lo + 63) / 64;
            const int64_t j = lo + (int64_t)lane * step;
            const int64_t oj = j < hi ? d[j].offset : INT64_MAX;
            const int c = __popcll(__ballot(oj <= e));
            if (c == 0) {                 // only when lo == 0: e lies before every tensor
                k = -1;
                if (lane == 0) s_next = oj;
                break;
            }
            const int64_t nhi = lo + (int64_t)c * step;
            lo = lo + (int64_t)(c - 1) * step;
            hi = nhi < hi ? nhi : hi;
        }
        if (k == -2) {
            // last round over [lo, hi] (at most 64 entries): every lane loads its
            // whole candidate, so the one found and the next offset reach the
            // block without another dependent load
            const int64_t j = lo + lane;
            const bool in_table = j < n;
            const zero_tensor_desc dj = in_table ? d[j] : zero_tensor_desc{nullptr, INT64_MAX, 0, 0};
            const int c = __popcll(__ballot(j < hi && dj.offset <= e));
            k = lo + c - 1;
            if (lane == c - 1) {
                s_ptr = (g_u16*)dj.ptr;
                s_off = dj.offset;
                s_numel = dj.numel;
            }
            if (lane == c) s_next = in_table ? dj.offset : INT64_MAX;
        }
        if (lane == 0) s_k = k;
    }
    __syncthreads();
    cur.k = s_k;
    cur.ptr = s_k >= 0 ? s_ptr : nullptr;
    cur.off = s_k >= 0 ? s_off : 0;
    cur.numel = s_k >= 0 ? s_numel : 0;
    cur.next = s_next;
}

// Copy between the flat buffer and the tensors the descriptors name
// (GATHER: tensors -> flat, zero where no tensor; else flat -> tensors).
// A lane owns one 8-element tile in each of the block's kFlatRows rows
// (aligned through the head split); a tile inside one tensor is "fast", the
// others go element by element.  The lane walks the descriptor table forward
// from the block's first tensor.  `flat` is only read when !GATHER.
//
// The tensor side of a fast tile is in general not 16-byte aligned (sh
// elements into its aligned chunk).  Consecutive lanes of a row hold
// consecutive tiles, so when the next lane's tile is the next 8 elements of
// the same tensor (known from the lane's own tile: 8 more elements remain in
// the tensor and the next lane is a vector lane of the row) the two tiles
// sit in consecutive memory, and the lanes share chunks:
//   gather: each lane loads its own first chunk and takes the second from
//     the next lane (a DPP lane shift); a lane whose next tile lies
//     elsewhere loads its second chunk itself;
//   scatter: each lane stores the aligned chunk that holds its last sh and
//     the next lane's first 8 - sh elements; a lane whose next tile lies
//     elsewhere stores its last sh elements one by one, and a lane whose
//     previous tile lies elsewhere stores its first 8 - sh (the same test,
//     seen from the other lane, so every element is written exactly once).
// Only the 16-byte chunks that hold a tile's own elements are read, and only
// its tensor's elements are written.  All loads of all rows are issued
// before the stores.  Block 0 also does the head and tail elements one per
// lane.
template <bool GATHER>
__device__ __forceinline__ void flat_copy(uint16_t* flat, const Split& s,
                                          const zero_tensor_desc* descs, int64_t n_descs) {
    const int64_t blk = block_id(s);
    const int64_t base = (s.aligned ? s.head : 0) + blk * (int64_t)kTile * kFlatRows;
    const int lane = threadIdx.x & 63;
    DescCursor cur;
    cur.d = descs;
    cur.n = n_descs;
    block_first_cursor(cur, descs, n_descs, blk == 0 ? 0 : base);
    bool fast[kFlatRows], next_ok[kFlatRows], prev_ok[kFlatRows];
    int64_t e0[kFlatRows];
    uintptr_t q[kFlatRows];                 // tensor-side address of a fast tile
#pragma unroll
    for (int t = 0; t < kFlatRows; ++t) {
        fast[t] = next_ok[t] = prev_ok[t] = false;
        q[t] = 0;
        const int64_t i = lane_tile<kFlatRows>(s, t);
        e0[t] = s.aligned ? s.head + i * kVec : i * kVec;
        const bool vec_lane = s.aligned && i < s.nvec;
        if (!vec_lane && (s.aligned || e0[t] >= s.count)) continue;
        cur.seek(e0[t]);
        const int64_t j0 = cur.index(e0[t]);
        if (vec_lane && j0 >= 0 && j0 + kVec <= cur.numel) {
            fast[t] = true;
            q[t] = (uintptr_t)(cur.ptr + j0);
            next_ok[t] = lane != 63 && j0 + 2 * kVec <= cur.numel && i + 1 < s.nvec;
            prev_ok[t] = lane != 0 && j0 >= kVec;
        } else if (vec_lane) {
            // a vector tile across a tensor boundary or over a gap: its flat
            // side is one aligned 16-byte chunk, so the tensor side goes
            // element by element with all loads before the stores (a load and
            // a store per element would serialise 8 memory round trips, the
            // two sides may alias)
            if (GATHER) {
                uint16_t h[kVec];
#pragma unroll
                for (int k = 0; k < kVec; ++k) {
                    cur.seek(e0[t] + k);
                    const int64_t j = cur.index(e0[t] + k);
                    h[k] = j >= 0 ? cur.ptr[j] : (uint16_t)0;
                }
                store_nt(flat + e0[t], pack8(h));
            } else {
                const u32x4 w = load_nt(flat + e0[t]);
#pragma unroll
                for (int k = 0; k < kVec; ++k) {
                    cur.seek(e0[t] + k);
                    const int64_t j = cur.index(e0[t] + k);
                    if (j >= 0) cur.ptr[j] = half_of(w, k);
                }
            }
        } else {
            for (int64_t e = e0[t]; e < e0[t] + kVec && e < s.count; ++e) {
                cur.seek(e);
                const int64_t j = cur.index(e);
                if (GATHER) flat[e] = j >= 0 ? cur.ptr[j] : (uint16_t)0;
                else if (j >= 0) cur.ptr[j] = flat[e];
            }
        }
    }
    u32x4 v[kFlatRows];
    if (GATHER) {
        u32x4 c1[kFlatRows];
#pragma unroll
        for (int t = 0; t < kFlatRows; ++t) {
            g_cu32x4* c = (g_cu32x4*)(q[t] & ~(uintptr_t)15);
            const int sh = (int)((q[t] & 15) >> 1);
            v[t] = u32x4{0, 0, 0, 0};
            c1[t] = u32x4{0, 0, 0, 0};
            if (fast[t]) v[t] = __builtin_nontemporal_load(c);
            if (fast[t] && sh != 0 && !next_ok[t]) c1[t] = __builtin_nontemporal_load(c + 1);
        }
#pragma unroll
        for (int t = 0; t < kFlatRows; ++t) {
            u32x4 nx;
#pragma unroll
            for (int w = 0; w < 4; ++w) nx[w] = from_next_lane(v[t][w]);
            if (next_ok[t]) c1[t] = nx;
            v[t] = window8(v[t], c1[t], (int)((q[t] & 15) >> 1));
        }
#pragma unroll
        for (int t = 0; t < kFlatRows; ++t)
            if (fast[t]) store_nt(flat + e0[t], v[t]);
    } else {
#pragma unroll
        for (int t = 0; t < kFlatRows; ++t) {
            v[t] = u32x4{0, 0, 0, 0};
            if (fast[t]) v[t] = load_nt(flat + e0[t]);
        }
#pragma unroll
        for (int t = 0; t < kFlatRows; ++t) {
            u32x4 nx;
#pragma unroll
            for (int w = 0; w < 4; ++w) nx[w] = from_next_lane(v[t][w]);
            if (!fast[t]) continue;
            g_u16* p = (g_u16*)q[t];
            const int m = (int)((q[t] & 15) >> 1);
            // whole 16-byte chunks go out non-temporally (written once; 0.84 ->
            // 0.79 ms for the 10,000-tensor write-back on MI355X)
            if (m == 0) {
                __builtin_nontemporal_store(v[t], (g_u32x4*)p);
                continue;
            }
            g_u16* c = (g_u16*)(q[t] & ~(uintptr_t)15);
            if (next_ok[t])
                __builtin_nontemporal_store(window8(v[t], nx, kVec - m), (g_u32x4*)(c + kVec));
            else store_elems(c + kVec, v[t], kVec - m, m);
            if (!prev_ok[t]) store_elems(p, v[t], 0, kVec - m);
        }
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
