// b3_kernels.hip - gfx950 kernels: chunk compression fused with the in-workgroup tree
// reduction (leaf), and the level reduction of chaining values (level).
//
// Page "BLAKE3 on GPU: 400x faster hashing" (qfminer.top):
//  - "Compression function" / "Kernel 1": one thread per 1 KiB chunk, 16 sequential
//    64-byte block compressions entirely in registers, CHUNK_START on the first block,
//    CHUNK_END on the last, the chunk index as counter.
//  - "Handling incomplete chunks": the last chunk may be shorter than 1 KiB, even shorter
//    than one block; its bytes past the end read as zero. Here a short chunk compresses
//    only its ceil(len/64) blocks (at least one), the last with its true byte count.
//  - "Merkle tree reduction": after the chunks, the workgroup reduces its chaining values
//    (CVs) level by level, halving the active lanes, with a barrier between levels; a
//    node count that is not a power of two yields perfect subtrees chained right to left.
//    Parents use counter 0, block length 64 and PARENT (plus KEYED_HASH in keyed mode).
//  - "Kernels 2 and 3": further levels reduce the per-workgroup roots; the final
//    compression of the whole tree carries ROOT.
//
// gfx950 design. Lane x of the workgroup owns tree node x; level l+1 node q is computed by
// lane q from level-l nodes 2q and 2q+1, so the active lanes stay packed at the bottom of
// the workgroup (dense waves) instead of spreading out. Keeping the node of an odd last
// position unchanged ("carry") at each level produces exactly the BLAKE3 shape: the left
// child of every node is then a complete power-of-two subtree and at least as large as
// the right one. Several independent segments (batch mode) share one workgroup by
// sitting at lane offsets aligned to the next power of two of their size, so that the
// same pairing never mixes two segments.
#include "b3_device.h"
#include "b3_kernels.h"

namespace b3g {
namespace {

__device__ __forceinline__ uint32_t ceil_log2(uint32_t n) {
    return n <= 1 ? 0u : 32u - static_cast<uint32_t>(__builtin_clz(n - 1));
}

// Word at byte offset `off` of a chunk holding `len` valid bytes; bytes at or past `len`
// read as zero and are never loaded.
__device__ __forceinline__ uint32_t load_word_bounded(const uint8_t *p, uint32_t off, uint32_t len) {
    if (off + 4 <= len) return *reinterpret_cast<const uint32_t *>(p + off);
    uint32_t w = 0;
    for (uint32_t k = 0; k < 4; ++k)
        if (off + k < len) w |= static_cast<uint32_t>(p[off + k]) << (8 * k);
    return w;
}

// Full 1 KiB chunk (16-byte aligned): the next block's four 16-byte loads are issued
// before the current block is compressed, so their latency hides behind ~680 VALU ops.
__device__ __forceinline__ void hash_full_chunk(uint32_t (&cv)[8], const uint8_t *chunk, uint32_t ctr_lo,
                                                uint32_t ctr_hi, uint32_t mode, uint32_t end_flags) {
    const uint4 *p = reinterpret_cast<const uint4 *>(chunk);
    uint4 q0 = p[0], q1 = p[1], q2 = p[2], q3 = p[3];
    for (uint32_t b = 0; b < kBlocksPerChunk; ++b) {
        const uint32_t m[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                                q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
        if (b + 1 < kBlocksPerChunk) {
            p += 4;
            q0 = p[0];
            q1 = p[1];
            q2 = p[2];
            q3 = p[3];
        }
        const uint32_t flags =
            mode | (b == 0 ? kChunkStart : 0u) | (b + 1 == kBlocksPerChunk ? end_flags : 0u);
        compress(cv, m, ctr_lo, ctr_hi, kBlockBytes, flags);
    }
}

// Chunk of `len` < 1024 bytes (only the last chunk of a message, or the empty message):
// max(1, ceil(len/64)) blocks, the last one of length len - 64*(blocks-1).
__device__ void hash_short_chunk(uint32_t (&cv)[8], const uint8_t *chunk, uint32_t len, uint32_t ctr_lo,
                                 uint32_t ctr_hi, uint32_t mode, uint32_t end_flags) {
    const uint32_t nb = len == 0 ? 1u : (len + kBlockBytes - 1) / kBlockBytes;
    for (uint32_t b = 0; b < kBlocksPerChunk; ++b) {
        if (b < nb) {
            const uint32_t off = b * kBlockBytes;
            uint32_t m[16];
#pragma unroll
            for (int w = 0; w < 16; ++w) m[w] = load_word_bounded(chunk, off + 4 * w, len);
            const bool last = b + 1 == nb;
            const uint32_t flags = mode | (b == 0 ? kChunkStart : 0u) | (last ? end_flags : 0u);
            compress(cv, m, ctr_lo, ctr_hi, last ? len - off : kBlockBytes, flags);
        }
    }
}

// One chunk per lane. Waves whose chunks are all full take the prefetching path; the
// (at most one per message) wave holding a short chunk takes the bounded path.
__device__ __forceinline__ void hash_chunk(uint32_t (&cv)[8], bool has_chunk, const uint8_t *chunk,
                                           uint32_t len, uint64_t counter, uint32_t mode, bool root) {
    const uint32_t lo = static_cast<uint32_t>(counter), hi = static_cast<uint32_t>(counter >> 32);
    const uint32_t end_flags = kChunkEnd | (root ? kRoot : 0u);
    if (__ballot(has_chunk && len != kChunkBytes) == 0) {
        if (has_chunk) hash_full_chunk(cv, chunk, lo, hi, mode, end_flags);
    } else {
        if (has_chunk) hash_short_chunk(cv, chunk, len, lo, hi, mode, end_flags);
    }
}

__device__ __forceinline__ void store_digest(uint8_t *out, const uint32_t (&cv)[8]) {
#pragma unroll
    for (int w = 0; w < 8; ++w)
#pragma unroll
        for (int k = 0; k < 4; ++k) out[4 * w + k] = static_cast<uint8_t>(cv[w] >> (8 * k));
}

__device__ __forceinline__ void store_cv(uint32_t *dst, const uint32_t (&cv)[8]) {
    uint4 *d = reinterpret_cast<uint4 *>(dst);
    d[0] = make_uint4(cv[0], cv[1], cv[2], cv[3]);
    d[1] = make_uint4(cv[4], cv[5], cv[6], cv[7]);
}

__device__ __forceinline__ void load_cv(uint32_t (&cv)[8], const uint32_t *src) {
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
    const uint4 a = s[0], b = s[1];
    cv[0] = a.x, cv[1] = a.y, cv[2] = a.z, cv[3] = a.w;
    cv[4] = b.x, cv[5] = b.y, cv[6] = b.z, cv[7] = b.w;
}

// ---- segment descriptions ------------------------------------------------------------

// Single message: the workgroup holds one segment of `n` nodes at lane 0.
struct SingleSegs {
    uint32_t n;
    bool whole;  // the segment is the whole message: its top compression carries ROOT
    uint32_t key[8];
    uint32_t mode_flag;
    uint32_t *cv_out;
    uint8_t *digest;

    __device__ int seg_of(uint32_t pos) const { return pos < n ? 0 : -1; }
    __device__ uint32_t start(int) const { return 0; }
    __device__ uint32_t count(int) const { return n; }
    __device__ bool final(int) const { return whole; }
    __device__ uint32_t mode() const { return mode_flag; }
    __device__ void key_words(int, uint32_t (&kw)[8]) const {
#pragma unroll
        for (int w = 0; w < 8; ++w) kw[w] = key[w];
    }
    __device__ void emit(int, const uint32_t (&cv)[8]) const {
        if (whole) store_digest(digest, cv);
        else store_cv(cv_out + 8ull * blockIdx.x, cv);
    }
};

// Batch: segments of this workgroup staged in LDS, plus the lane -> segment map.
struct BatchSegs {
    const Seg *seg;        // LDS
    const int *seg_of_pos; // LDS, one entry per lane position
    const uint32_t *keys;  // global, nullptr for default mode
    uint32_t *cv_out;
    uint8_t *digests;

    __device__ int seg_of(uint32_t pos) const { return seg_of_pos[pos]; }
    __device__ uint32_t start(int s) const { return seg_lane(seg[s].info); }
    __device__ uint32_t count(int s) const { return seg_count(seg[s].info); }
    __device__ bool final(int s) const { return seg_final(seg[s].info); }
    __device__ uint32_t mode() const { return keys ? kKeyedHash : 0u; }
    __device__ void key_words(int s, uint32_t (&kw)[8]) const {
        if (keys) {
            load_cv(kw, keys + 8ull * seg[s].msg);
        } else {
#pragma unroll
            for (int w = 0; w < 8; ++w) kw[w] = kIV[w];
        }
    }
    __device__ void emit(int s, const uint32_t (&cv)[8]) const {
        if (final(s)) store_digest(digests + 32ull * seg[s].msg, cv);
        else store_cv(cv_out + 8ull * seg[s].dst, cv);
    }
};

// Loads this workgroup's segments into LDS and maps every lane position to its segment
// (or -1). Segments are sorted by lane start.
template <uint32_t C>
__device__ __forceinline__ void stage_segments(const uint32_t *wg_first_seg, const Seg *segs, Seg *s_seg,
                                               int *s_seg_of) {
    const uint32_t lane = threadIdx.x;
    const uint32_t first = wg_first_seg[blockIdx.x];
    const uint32_t nseg = wg_first_seg[blockIdx.x + 1] - first;
    for (uint32_t i = lane; i < nseg; i += C) s_seg[i] = segs[first + i];
    __syncthreads();
    // largest i with start(i) <= lane
    uint32_t lo = 0, hi = nseg;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (seg_lane(s_seg[mid].info) <= lane) lo = mid;
        else hi = mid;
    }
    int s = -1;
    if (nseg > 0) {
        const uint32_t info = s_seg[lo].info;
        if (lane >= seg_lane(info) && lane < seg_lane(info) + seg_count(info)) s = static_cast<int>(lo);
    }
    s_seg_of[lane] = s;
    __syncthreads();
}

// The fused partial Merkle reduction. On entry lane x holds the level-0 node x in `cv`
// (if it belongs to a segment). Each segment's result is emitted by the lane that
// computes it, at the level where the segment reaches a single node.
template <uint32_t C, class Segs>
__device__ __forceinline__ void tree_reduce(const uint32_t (&cv)[8], const Segs &sg, uint32_t levels,
                                            uint32_t (*buf)[8][C]) {
    const uint32_t lane = threadIdx.x;
    const int s0 = sg.seg_of(lane);
    if (s0 >= 0) {
#pragma unroll
        for (int w = 0; w < 8; ++w) buf[0][w][lane] = cv[w];
        if (sg.count(s0) == 1) sg.emit(s0, cv);
    }
    for (uint32_t l = 0; l < levels; ++l) {
        __syncthreads();
        const uint32_t pos = lane << (l + 1);  // first leaf position under output node `lane`
        if (pos >= C) continue;
        const int s = sg.seg_of(pos);
        if (s < 0) continue;
        const uint32_t start = sg.start(s), n = sg.count(s), r = ceil_log2(n);
        if (l >= r) continue;  // segment already reduced to one node
        const uint32_t(*src)[C] = buf[l & 1];
        uint32_t node[8];
        const bool has_right = (((2 * lane + 1) << l) - start) < n;
        if (has_right) {
            uint32_t m[16];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const uint2 pr = *reinterpret_cast<const uint2 *>(&src[w][2 * lane]);
                m[w] = pr.x;
                m[w + 8] = pr.y;
            }
            sg.key_words(s, node);
            const uint32_t flags = sg.mode() | kParent | (sg.final(s) && l + 1 == r ? kRoot : 0u);
            compress(node, m, 0, 0, kBlockBytes, flags);
        } else {
#pragma unroll
            for (int w = 0; w < 8; ++w) node[w] = src[w][2 * lane];
        }
#pragma unroll
        for (int w = 0; w < 8; ++w) buf[(l + 1) & 1][w][lane] = node[w];
        if (l + 1 == r) sg.emit(s, node);
    }
}

// ---- kernels ---------------------------------------------------------------------------

__global__ __launch_bounds__(kLeafLanes) void leaf_single_kernel(SingleLeafArgs a) {
    __shared__ uint32_t buf[2][8][kLeafLanes];
    const uint32_t lane = threadIdx.x;
    const uint64_t first = static_cast<uint64_t>(blockIdx.x) * kLeafLanes;
    const uint64_t left = a.n_chunks - first;
    const uint32_t n_wg = left < kLeafLanes ? static_cast<uint32_t>(left) : kLeafLanes;
    const bool has_chunk = lane < n_wg;
    const uint64_t chunk = first + lane;
    uint32_t len = 0;
    if (has_chunk) {
        const uint64_t rem = a.len - chunk * kChunkBytes;  // len == 0 only for the empty message
        len = a.len == 0 ? 0u : (rem < kChunkBytes ? static_cast<uint32_t>(rem) : kChunkBytes);
    }
    const bool whole = a.may_root && gridDim.x == 1;
    uint32_t cv[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) cv[w] = a.key[w];
    hash_chunk(cv, has_chunk, a.in + chunk * kChunkBytes, len, a.chunk_base + chunk, a.mode,
               whole && a.n_chunks == 1);
    SingleSegs sg{n_wg, whole, {a.key[0], a.key[1], a.key[2], a.key[3], a.key[4], a.key[5], a.key[6], a.key[7]},
                  a.mode, a.cv_out, a.digest};
    tree_reduce<kLeafLanes>(cv, sg, ceil_log2(n_wg), buf);
}

__global__ __launch_bounds__(kLevelLanes) void level_single_kernel(SingleLevelArgs a) {
    __shared__ uint32_t buf[2][8][kLevelLanes];
    const uint32_t lane = threadIdx.x;
    const uint64_t first = static_cast<uint64_t>(blockIdx.x) * kLevelLanes;
    const uint64_t left = a.m - first;
    const uint32_t n_wg = left < kLevelLanes ? static_cast<uint32_t>(left) : kLevelLanes;
    uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (lane < n_wg) load_cv(cv, a.cv_in + 8 * (first + lane));
    SingleSegs sg{n_wg, gridDim.x == 1,
                  {a.key[0], a.key[1], a.key[2], a.key[3], a.key[4], a.key[5], a.key[6], a.key[7]},
                  a.mode, a.cv_out, a.digest};
    tree_reduce<kLevelLanes>(cv, sg, ceil_log2(n_wg), buf);
}

__global__ __launch_bounds__(kLeafLanes) void leaf_batch_kernel(BatchLeafArgs a) {
    __shared__ uint32_t buf[2][8][kLeafLanes];
    __shared__ Seg s_seg[kLeafLanes];
    __shared__ int s_seg_of[kLeafLanes];
    stage_segments<kLeafLanes>(a.wg_first_seg, a.segs, s_seg, s_seg_of);
    const uint32_t lane = threadIdx.x;
    const int s = s_seg_of[lane];
    const bool has_chunk = s >= 0;
    BatchSegs sg{s_seg, s_seg_of, a.keys, a.cv_out, a.digests};
    uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint8_t *ptr = a.base;
    uint32_t len = 0;
    uint64_t chunk = 0;
    bool root = false;
    if (has_chunk) {
        const Seg g = s_seg[s];
        chunk = g.first + (lane - seg_lane(g.info));
        const uint64_t mlen = a.msg_len[g.msg];
        const uint64_t rem = mlen - chunk * kChunkBytes;
        len = mlen == 0 ? 0u : (rem < kChunkBytes ? static_cast<uint32_t>(rem) : kChunkBytes);
        ptr = a.base + a.msg_off[g.msg] + chunk * kChunkBytes;
        root = seg_final(g.info) && seg_count(g.info) == 1;
        sg.key_words(s, cv);
    }
    hash_chunk(cv, has_chunk, ptr, len, chunk, sg.mode(), root);
    tree_reduce<kLeafLanes>(cv, sg, a.wg_levels[blockIdx.x], buf);
}

__global__ __launch_bounds__(kLevelLanes) void level_batch_kernel(BatchLevelArgs a) {
    __shared__ uint32_t buf[2][8][kLevelLanes];
    __shared__ Seg s_seg[kLevelLanes];
    __shared__ int s_seg_of[kLevelLanes];
    stage_segments<kLevelLanes>(a.wg_first_seg, a.segs, s_seg, s_seg_of);
    const uint32_t lane = threadIdx.x;
    const int s = s_seg_of[lane];
    uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (s >= 0) {
        const Seg g = s_seg[s];
        load_cv(cv, a.cv_in + 8ull * (g.first + (lane - seg_lane(g.info))));
    }
    BatchSegs sg{s_seg, s_seg_of, a.keys, a.cv_out, a.digests};
    tree_reduce<kLevelLanes>(cv, sg, a.wg_levels[blockIdx.x], buf);
}

}  // namespace

hipError_t launch_single_leaf(const SingleLeafArgs &a, uint32_t grid, hipStream_t s) {
    hipLaunchKernelGGL(leaf_single_kernel, dim3(grid), dim3(kLeafLanes), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_single_level(const SingleLevelArgs &a, uint32_t grid, hipStream_t s) {
    hipLaunchKernelGGL(level_single_kernel, dim3(grid), dim3(kLevelLanes), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_batch_leaf(const BatchLeafArgs &a, uint32_t grid, hipStream_t s) {
    hipLaunchKernelGGL(leaf_batch_kernel, dim3(grid), dim3(kLeafLanes), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_batch_level(const BatchLevelArgs &a, uint32_t grid, hipStream_t s) {
    hipLaunchKernelGGL(level_batch_kernel, dim3(grid), dim3(kLevelLanes), 0, s, a);
    return hipGetLastError();
}

}  // namespace b3g
