// zero_common.h -- internal to the library: tile geometry, 128-bit memory
// helpers, pointer-alignment split and the typed launcher shared by the
// owner-step kernels (zero_shard.hip) and the flat copy kernels
// (zero_flat.hip).  Each translation unit gets its own internal copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "zero_shard.h"

namespace {

constexpr int kThreads = 256;          // 4 wave64s per block
constexpr int kVec = 8;                // elements per lane tile (one 128-bit 16-bit access)
constexpr int kTile = kThreads * kVec; // elements per block and lane tile
constexpr int kFold = 2048;            // partials folded per block per fold pass
constexpr int kFinal = 16384;          // partials the one-block final pass takes
constexpr int kMaxStreamBlocks = 256 * 8;  // grid-stride kernels off the hot path
// A launch's total thread count must fit in 32 bits (the dispatch packet's
// grid size; HIP truncates it silently beyond that), so tile kernels are
// launched in pieces of at most this many blocks (34.4e9 elements at one lane
// tile per lane); Split::blk0 carries the piece's first block.
constexpr int64_t kMaxLaunchBlocks = (int64_t(1) << 32) / kThreads - 1;
// LDS per CU on gfx950.  Dynamic LDS is used to cap how many blocks of a
// streaming kernel share a CU (lds_for_blocks).
constexpr unsigned kLdsPerCU = 160 * 1024;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// How the elements of a call map onto tiles.  With `aligned`, lanes run the
// 128-bit path over [head, head + 8*nvec) and block 0 also does the `head`
// leading and the < 8 trailing elements one by one; otherwise every lane
// walks its 8 elements with 16/32-bit accesses.
struct Split {
    int64_t head, nvec, count;
    int64_t blk0;      // global index of the launch's first block
    int aligned;
};

// ---------------------------------------------------------------- memory ----
__device__ __forceinline__ u32x4 load_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store_nt(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x2 load_nt_b64(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ void store_nt_b64(uint16_t* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ u32x4 load_b128(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store_b128(uint16_t* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ f32x4 load_f4(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void store_f4(float* p, f32x4 v) {
    *reinterpret_cast<f32x4*>(p) = v;
}
// One wave instruction of a direct global -> LDS copy (gfx950
// global_load_lds_dwordx4): lane l moves the 16 bytes at its own `src` to
// lds + 16 l, so 64 lanes fill 1 KiB of LDS without going through VGPRs.
// `lds` must be the same for every lane of the wave.  NT selects a
// non-temporal (streaming) load.  The data may be read from LDS once the
// wave's vector-memory counter has drained.
template <bool NT>
__device__ __forceinline__ void load_to_lds(const void* src, char* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, NT ? 2 : 0);
}
__device__ __forceinline__ uint16_t half_of(u32x4 w, int k) {
    return (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu));
}
__device__ __forceinline__ uint16_t half_of2(u32x2 w, int k) {
    return (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu));
}
__device__ __forceinline__ u32x2 pack4(const uint16_t* h) {
    u32x2 w;
    w[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    w[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    return w;
}
__device__ __forceinline__ u32x4 pack8(const uint16_t* h) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)h[2 * q] | ((uint32_t)h[2 * q + 1] << 16);
    return w;
}
// Global block index of a tile kernel launched in pieces.
__device__ __forceinline__ int64_t block_id(const Split& s) {
    return s.blk0 + (int64_t)blockIdx.x;
}
// Lane tile of lane threadIdx.x in the t-th of TPL block-wide rows of lane
// tiles that block block_id(s) owns: consecutive lanes, consecutive tiles.
template <int TPL = 1>
__device__ __forceinline__ int64_t lane_tile(const Split& s, int t = 0) {
    return (block_id(s) * TPL + t) * kThreads + threadIdx.x;
}

// ------------------------------------------------------------ host -------
inline bool valid_dtype(int32_t dt) { return dt == ZERO_FP16 || dt == ZERO_BF16; }

// Leading elements to handle one by one so that every pointer is 16-byte
// aligned for the vector body, or -1 when no such count exists.
inline int64_t vector_head(const void* const* p16, int n16, const void* const* p32, int n32) {
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

inline Split split_for(int64_t head, int64_t count) {
    Split s;
    s.count = count;
    s.blk0 = 0;
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

// Blocks of a tile kernel whose lanes take TPL lane tiles each, at least one.
inline int64_t tile_blocks(const Split& s, int tpl = 1) {
    const int64_t lanes = s.aligned ? s.nvec : (s.count + kVec - 1) / kVec;
    const int64_t per = (int64_t)kThreads * tpl;
    const int64_t b = (lanes + per - 1) / per;
    return b < 1 ? 1 : b;
}

// Upper bound of tile_blocks over all alignments of `count` elements.
inline int64_t max_tile_blocks(int64_t count) {
    return (count + kTile - 1) / kTile + 1;
}

// Dynamic LDS bytes that leave room for exactly `b` resident blocks per CU
// (0: no cap).  Streaming kernels with many concurrent HBM streams run
// faster on MI355X with fewer waves in flight: fewer DRAM rows are open at
// once, while enough bytes stay in flight to cover the latency.
inline unsigned lds_for_blocks(int b) {
    return b >= 8 ? 0u : kLdsPerCU / (unsigned)(b + 1) + 2048u;
}

// Launches `kernel` on `grid` blocks of `threads` lanes with `lds` bytes of
// dynamic LDS, its arguments converted to the kernel's parameter types, and
// returns this launch's own status (not a stale thread-local one).
template <typename... KArgs, typename... Args>
inline int launch_shape(void (*kernel)(KArgs...), int64_t grid, int threads, unsigned lds,
                        hipStream_t stream, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    if (grid < 1 || grid > kMaxLaunchBlocks) return ZERO_ERANGE;
    std::tuple<KArgs...> packed(static_cast<KArgs>(args)...);
    void* ptrs[sizeof...(KArgs)];
    int i = 0;
    std::apply([&](auto&... a) { ((ptrs[i++] = (void*)&a), ...); }, packed);
    const hipError_t err = hipLaunchKernel((const void*)kernel, dim3((unsigned)grid),
                                           dim3((unsigned)threads), ptrs, lds, stream);
    return err == hipSuccess ? ZERO_OK : ZERO_EDEVICE;
}

// A launch of 256-lane blocks (every kernel but the one-thread control update).
template <typename... KArgs, typename... Args>
inline int launch(void (*kernel)(KArgs...), int64_t grid, unsigned lds, hipStream_t stream,
                  Args... args) {
    return launch_shape(kernel, grid, kThreads, lds, stream, args...);
}

// Runs a tile kernel over `blocks` blocks as launches of at most
// kMaxLaunchBlocks, in order on one stream: go(piece, grid) launches one
// piece, whose Split has blk0 set.
template <typename F>
inline int launch_pieces(const Split& s, int64_t blocks, F&& go) {
    for (int64_t b0 = 0; b0 < blocks; b0 += kMaxLaunchBlocks) {
        Split piece = s;
        piece.blk0 = b0;
        const int64_t g = blocks - b0 < kMaxLaunchBlocks ? blocks - b0 : kMaxLaunchBlocks;
        const int rc = go(piece, g);
        if (rc != ZERO_OK) return rc;
    }
    return ZERO_OK;
}

}  // namespace
