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
// gfx950 design. In the leaf kernel each lane hashes K consecutive chunks (K = 1, 2 or 4,
// chosen by input size) and folds them into one subtree node in registers, so the first
// log2(K) tree levels cost no cross-lane traffic and the lane-sparse top of the workgroup
// tree is paid once per 256*K chunks. Lane x of the workgroup owns tree node x; level l+1
// node q is computed by lane q from level-l nodes 2q and 2q+1, so the active lanes stay
// packed at the bottom of the workgroup (dense waves) instead of spreading out. Keeping
// the node of an odd last position unchanged ("carry") at each level produces exactly the
// BLAKE3 shape: the left child of every node is then a complete power-of-two subtree and
// at least as large as the right one. Several independent segments (batch mode) share
// one workgroup by sitting at lane offsets aligned to the next power of two of their
// size, so that the same pairing never mixes two segments.
#include <utility>
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

struct Block {
    uint4 q0, q1, q2, q3;
};

__device__ __forceinline__ void compress_block(uint32_t (&cv)[8], const Block &k, uint32_t lo, uint32_t hi,
                                               uint32_t flags, uint32_t block_len = kBlockBytes) {
    const uint32_t m[16] = {k.q0.x, k.q0.y, k.q0.z, k.q0.w, k.q1.x, k.q1.y, k.q1.z, k.q1.w,
                            k.q2.x, k.q2.y, k.q2.z, k.q2.w, k.q3.x, k.q3.y, k.q3.z, k.q3.w};
    compress(cv, m, lo, hi, block_len, flags);
}

__device__ __forceinline__ Block load_block(const uint4 *p) { return Block{p[0], p[1], p[2], p[3]}; }

// v <- the state after block k, chained from state s (see compress_chained).
__device__ __forceinline__ void compress_block_chained(const uint32_t (&s)[16], const Block &k, uint32_t lo, uint32_t hi,
                                                       uint32_t flags, uint32_t (&v)[16]) {
    const uint32_t m[16] = {k.q0.x, k.q0.y, k.q0.z, k.q0.w, k.q1.x, k.q1.y, k.q1.z, k.q1.w,
                            k.q2.x, k.q2.y, k.q2.z, k.q2.w, k.q3.x, k.q3.y, k.q3.z, k.q3.w};
    compress_chained(s, m, lo, hi, kBlockBytes, flags, v);
}

// Issue-priority turns for waves that share a SIMD (Turns below). The SIMD issues from the
// highest-priority wave that is ready, and among equals from the oldest, so of two waves
// that start together the older one runs its whole chunk with the younger one only taking
// the cycles it leaves idle, and the younger then runs alone, at the rate of a lone wave,
// for most of its own chunk. Stepping a wave's priority down from 3 to 0 as it passes
// blocks 8, 12 and 14 of its chunk lets the waves take turns (over eight blocks, then four,
// then two), so both keep the SIMD busy until they end, close together: the last phase,
// where the older wave goes first again, is two blocks long (steps at 4, 8 and 12 left four,
// and measured slower).
__device__ __forceinline__ void turn_priority_at(uint32_t b) {
    if (b == 8) __builtin_amdgcn_s_setprio(2);
    else if (b == 12) __builtin_amdgcn_s_setprio(1);
    else if (b == 14) __builtin_amdgcn_s_setprio(0);
}

// Full 1 KiB chunk with per-lane 16-byte loads (16-byte aligned). Blocks are handled in
// pairs with two register sets, so the loads of a block are issued ahead of its
// compression and no registers are copied between iterations; the reload of the even set
// is unconditional (the last iteration re-reads block 14, which is in cache) so that the
// loop carries no conditional register values. Between blocks the state stays unfolded
// (compress_chained), alternating between two arrays; the first block starts from the
// state (cv, 0), whose fold is cv. `end_flags` go on the last block (CHUNK_END, plus ROOT
// when the chunk is the whole message).
template <bool Turns = false>
__device__ __forceinline__ void hash_full_chunk(uint32_t (&cv)[8], const uint8_t *chunk, uint32_t ctr_lo,
                                                uint32_t ctr_hi, uint32_t mode, uint32_t end_flags) {
    const uint4 *p = reinterpret_cast<const uint4 *>(chunk);
    // the state after an even block (st) and after an odd one (su); st starts as a state
    // whose fold is the chaining value the chunk starts from
    uint32_t st[16], su[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) st[i] = cv[i], st[i + 8] = 0;
    Block even = load_block(p);
    if (Turns) __builtin_amdgcn_s_setprio(3);
    for (uint32_t b = 0; b < kBlocksPerChunk; b += 2) {
        if (Turns) turn_priority_at(b);
        const Block odd = load_block(p + 4 * (b + 1));
        compress_block_chained(st, even, ctr_lo, ctr_hi, mode | (b == 0 ? kChunkStart : 0u), su);
        const uint32_t next = b + 2 < kBlocksPerChunk ? b + 2 : kBlocksPerChunk - 2;
        even = load_block(p + 4 * next);
        compress_block_chained(su, odd, ctr_lo, ctr_hi, mode | (b + 2 == kBlocksPerChunk ? end_flags : 0u), st);
    }
    fold_state(cv, st);
}

// The same chunk hash with a whole 128-byte line (two blocks) of loads in flight ahead
// of the compressions: the loads of blocks b + 2 and b + 3 are issued before blocks b and
// b + 1 are compressed, so that each block's data has two compressions to arrive. The
// scheduling barriers keep the compiler from sinking the loads towards their use (the
// input is read-only, so a memory clobber would not hold them). It takes 32 more
// registers; it is used where waves have few neighbours on their SIMD to hide a load
// behind (single messages and uniform batches: 64 MiB 44.4 -> 42.5 us, 1 GiB 360 -> 355
// us, 4 GiB + 1000 B 1.370 -> 1.360 ms, measured on MI355X), not for the batches planned
// into a task table, where it measured slower (256 ragged messages 77.5 -> 79.0 us).
// ea, oa: on entry blocks 0 and 1 of this chunk (loaded by the caller); on exit blocks 0
// and 1 at `next`, loaded during the chunk's last blocks, so that a lane folding several
// chunks never waits at a chunk boundary (`next` is the lane's next chunk, or any readable
// 128 bytes).
__device__ __forceinline__ void hash_full_chunk_line_ahead(uint32_t (&cv)[8], const uint8_t *chunk, uint32_t ctr_lo,
                                                           uint32_t ctr_hi, uint32_t mode, uint32_t end_flags,
                                                           Block &ea, Block &oa, const uint8_t *next) {
    const uint4 *p = reinterpret_cast<const uint4 *>(chunk);
    const uint4 *pn = reinterpret_cast<const uint4 *>(next);
    uint32_t st[16], su[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) st[i] = cv[i], st[i + 8] = 0;
    for (uint32_t b = 0; b < kBlocksPerChunk; b += 4) {
        const Block eb = load_block(p + 4 * (b + 2)), ob = load_block(p + 4 * (b + 3));
        __builtin_amdgcn_sched_barrier(0);
        compress_block_chained(st, ea, ctr_lo, ctr_hi, mode | (b == 0 ? kChunkStart : 0u), su);
        compress_block_chained(su, oa, ctr_lo, ctr_hi, mode, st);
        // blocks b + 4 and b + 5; in the last iteration blocks 0 and 1 at `next` (a select
        // of the address, so that the loop carries no conditional register values)
        const uint4 *q = b + 4 < kBlocksPerChunk ? p + 4 * (b + 4) : pn;
        ea = load_block(q);
        oa = load_block(q + 4);
        __builtin_amdgcn_sched_barrier(0);
        compress_block_chained(st, eb, ctr_lo, ctr_hi, mode, su);
        compress_block_chained(su, ob, ctr_lo, ctr_hi, mode | (b + 4 == kBlocksPerChunk ? end_flags : 0u), st);
    }
    fold_state(cv, st);
}

// Sixteen zero bytes in device memory: the source of every load of a chunk piece that
// lies past the chunk's end, so that those loads need no branch and never leave the
// chunk's valid bytes.
__device__ __attribute__((aligned(16))) uint8_t g_zero_piece[16];

// The 16-byte piece of a chunk that holds its last byte without being whole (the piece at
// len & ~15 when len is not a multiple of 16; zeros otherwise), by byte loads from the
// chunk's valid bytes or the zero piece.
__device__ __forceinline__ uint4 load_tail_piece(const uint8_t *chunk, uint32_t len) {
    const uint32_t off = len & ~15u;
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (uint32_t k = 0; k < 16; ++k) {
        const uint8_t *src = off + k < len ? chunk + off + k : g_zero_piece + k;
        w[k / 4] |= static_cast<uint32_t>(*src) << (8 * (k % 4));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 16-byte piece at byte `at` of a chunk holding `len` valid bytes when it lies wholly
// inside them, else zeros (loaded from the zero piece, so that the load needs no branch).
__device__ __forceinline__ uint4 load_piece_or_zero(const uint8_t *chunk, uint32_t at, uint32_t len) {
    return *reinterpret_cast<const uint4 *>(at + 16 <= len ? chunk + at : g_zero_piece);
}

__device__ __forceinline__ Block load_block_or_zero(const uint8_t *chunk, uint32_t off, uint32_t len) {
    return Block{load_piece_or_zero(chunk, off, len), load_piece_or_zero(chunk, off + 16, len),
                 load_piece_or_zero(chunk, off + 32, len), load_piece_or_zero(chunk, off + 48, len)};
}

// Chunk of `len` <= 1024 bytes with per-lane loads that never read past `len`:
// max(1, ceil(len/64)) blocks, the last one of length len - 64*(blocks-1). The loads are
// branch-free: a 16-byte piece wholly inside the chunk is one 16-byte load, a piece past
// the end is loaded from the zero piece, and the piece holding the last byte, loaded once
// (load_tail_piece), is substituted at its offset. (Bounded loads with branches cost a
// quarter more VALU instructions and three hundred scalar ones per block.) Each block is
// loaded when its compression starts, which keeps the kernels that hash single messages
// at their register count: their short chunks are a message's last.
__device__ void hash_short_chunk(uint32_t (&cv)[8], const uint8_t *chunk, uint32_t len, uint32_t ctr_lo,
                                 uint32_t ctr_hi, uint32_t mode, uint32_t end_flags) {
    const uint32_t nb = len == 0 ? 1u : (len + kBlockBytes - 1) / kBlockBytes;
    const uint4 tail = load_tail_piece(chunk, len);
    const uint32_t tail_off = len & ~15u;
    for (uint32_t b = 0; b < nb; ++b) {
        const uint32_t off = b * kBlockBytes;
        uint4 q[4];
#pragma unroll
        for (uint32_t p = 0; p < 4; ++p) {
            q[p] = load_piece_or_zero(chunk, off + 16 * p, len);
            if (off + 16 * p == tail_off) q[p] = tail;
        }
        const bool last = b + 1 == nb;
        const uint32_t flags = mode | (b == 0 ? kChunkStart : 0u) | (last ? end_flags : 0u);
        compress_block(cv, Block{q[0], q[1], q[2], q[3]}, ctr_lo, ctr_hi, flags, last ? len - off : kBlockBytes);
    }
}

// The same chunk hash with each block's loads issued while the block before it is
// compressed (16 more registers), for waves that hold only message ends and often run
// alone on their SIMD at the end of a batch's grid, where a load per block would wait
// for memory every time. Every block but the last lies wholly inside the chunk; a lane's
// loop runs its own block count and the wave's last blocks are compressed together, with
// the piece holding the last byte substituted.
template <bool Turns = false>
__device__ void hash_short_chunk_ahead(uint32_t (&cv)[8], const uint8_t *chunk, uint32_t len, uint32_t ctr_lo,
                                       uint32_t ctr_hi, uint32_t mode, uint32_t end_flags) {
    const uint32_t nb = len == 0 ? 1u : (len + kBlockBytes - 1) / kBlockBytes;
    const uint4 tail = load_tail_piece(chunk, len);
    const uint32_t tail_off = len & ~15u;
    Block cur = load_block_or_zero(chunk, 0, len);
    if (Turns) __builtin_amdgcn_s_setprio(3);
    for (uint32_t b = 0; b + 1 < nb; ++b) {
        if (Turns) turn_priority_at(b);
        const Block next = load_block_or_zero(chunk, (b + 1) * kBlockBytes, len);
        compress_block(cv, cur, ctr_lo, ctr_hi, mode | (b == 0 ? kChunkStart : 0u));
        cur = next;
    }
    const uint32_t off = (nb - 1) * kBlockBytes;
    if (off == tail_off) cur.q0 = tail;
    if (off + 16 == tail_off) cur.q1 = tail;
    if (off + 32 == tail_off) cur.q2 = tail;
    if (off + 48 == tail_off) cur.q3 = tail;
    compress_block(cv, cur, ctr_lo, ctr_hi, mode | (nb == 1 ? kChunkStart : 0u) | end_flags, len - off);
}

constexpr uint32_t kLanes = kLeafLanes;
constexpr uint32_t kWaveLanes = 64;

// c <- parent(left, c): the two CVs as one 64-byte block, compressed from the key words
// with counter 0, block length 64 and PARENT (ROOT when `root`).
__device__ __forceinline__ void parent_left(uint32_t (&c)[8], const uint32_t (&left)[8], const uint32_t (&key)[8],
                                            uint32_t mode, bool root) {
    uint32_t m[16];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        m[w] = left[w];
        m[w + 8] = c[w];
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) c[w] = key[w];
    compress(c, m, 0, 0, kBlockBytes, mode | kParent | (root ? kRoot : 0u));
}

// Folds chunk k's CV `c` into the lane's pending subtrees. After chunk k the lane holds
// one complete subtree per set bit of k+1; chunk k's CV merges with the pending subtree
// of each size 2^lv for which bit lv of k is set (its left neighbours of equal size),
// which keeps every left subtree a complete power of two, at least as large as its
// right sibling. With K <= 4 a subtree waiting for a right sibling has 1 chunk (slot1c)
// or 2 chunks (slot2c); the slots are only ever named directly, so they stay in
// registers. `fin_k` is the index of the lane's last chunk when this node is the whole
// message (the merge that produces all of it carries ROOT), else K.
template <uint32_t K>
__device__ __forceinline__ void fold_chunk(uint32_t (&c)[8], uint32_t k, uint32_t (&slot1c)[8],
                                           uint32_t (&slot2c)[8], bool store, uint32_t fin_k,
                                           const uint32_t (&key)[8], uint32_t mode) {
    if (k & 1u) {
        parent_left(c, slot1c, key, mode, k == fin_k && k == 1);
        if (K > 2 && (k & 2u)) parent_left(c, slot2c, key, mode, k == fin_k && k == 3);
    }
    // both slots are written every time (value selects): a store to a conditionally chosen
    // slot would be merged into one store through a selected address, moving the slots
    // out of registers
    const bool to1 = store && !(k & 1u);
    const bool to2 = K > 2 && store && (k & 1u) && !(k & 2u);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        slot1c[w] = to1 ? c[w] : slot1c[w];
        slot2c[w] = to2 ? c[w] : slot2c[w];
    }
}

// Per-lane path (waves holding a short chunk or lanes with fewer than K chunks, i.e.
// the ends of messages): the lane's nl (1..K) consecutive chunks, starting at `ptr` with
// counter ctr0, reduced to one node, the BLAKE3 tree over nl leaves. Loads are
// per-lane and bounded by the byte count. The last chunk has last_len bytes (1024 unless
// it ends the message). `root`: this node is the whole message, so its final compression
// carries ROOT.
template <uint32_t K, bool Ahead = false, bool Turns = false>
__device__ __forceinline__ void lane_subtree(uint32_t (&c)[8], const uint8_t *ptr, uint32_t nl,
                                             uint32_t last_len, uint64_t ctr0, const uint32_t (&key)[8],
                                             uint32_t mode, bool root) {
    uint32_t slot1c[8], slot2c[8];
    const uint32_t fin_k = root ? nl - 1 : K;
    for (uint32_t k = 0; k < nl; ++k) {
#pragma unroll
        for (int w = 0; w < 8; ++w) c[w] = key[w];
        const uint64_t ctr = ctr0 + k;
        const uint32_t lo = static_cast<uint32_t>(ctr), hi = static_cast<uint32_t>(ctr >> 32);
        const uint32_t end_flags = kChunkEnd | (root && nl == 1 ? kRoot : 0u);
        const uint8_t *chunk = ptr + static_cast<uint64_t>(k) * kChunkBytes;
        const uint32_t len = k + 1 == nl ? last_len : kChunkBytes;
        if (Ahead) hash_short_chunk_ahead<Turns>(c, chunk, len, lo, hi, mode, end_flags);
        else hash_short_chunk(c, chunk, len, lo, hi, mode, end_flags);
        if (K > 1) fold_chunk<K>(c, k, slot1c, slot2c, k + 1 < nl, fin_k, key, mode);
    }
    // nl not a power of two (only 3 when K <= 4): the 2-chunk subtree on the left remains
    if (K > 2 && nl == 3) parent_left(c, slot2c, key, mode, root);
}

// ---- full waves, direct loads (default) ---------------------------------------------
// Every lane of the wave holds K full chunks. Each lane reads its own chunks with 16-byte
// loads; a lane starts at chunk (lane mod K) of its run and wraps around, so that at
// every step the 64 lanes read from K different 1 KiB offsets of their K KiB spans
// (with equal offsets every lane's line falls in the same cache set and channel and is
// evicted between the two blocks that share it). The chunk CVs wait in LDS slots, one
// column per lane (slot j, word w at slots[(j * 8 + w) * kLanes]), and are folded at the
// end, level by level: node i = parent(node 2i, node 2i+1). `root_flag` (ROOT or 0)
// marks the lane's node as the whole message: its last compression carries it.
// LineAhead: each chunk by hash_full_chunk_line_ahead rather than hash_full_chunk.
template <uint32_t K, bool LineAhead, bool Turns = false>
__device__ __forceinline__ void direct_subtree(uint32_t (&c)[8], const uint8_t *ptr, uint64_t ctr0,
                                               const uint32_t (&key)[8], uint32_t mode, uint32_t root_flag,
                                               uint32_t *slots) {
    const uint32_t rot = threadIdx.x % K;
    Block ea, oa;  // blocks 0 and 1 of the next chunk (line-ahead form)
    if (LineAhead) {
        const uint4 *p0 = reinterpret_cast<const uint4 *>(ptr + static_cast<uint64_t>(rot) * kChunkBytes);
        ea = load_block(p0);
        oa = load_block(p0 + 4);
    }
    for (uint32_t step = 0; step < K; ++step) {
        const uint32_t k = (step + rot) % K;
#pragma unroll
        for (int w = 0; w < 8; ++w) c[w] = key[w];
        const uint64_t ctr = ctr0 + k;
        const uint8_t *chunk = ptr + static_cast<uint64_t>(k) * kChunkBytes;
        if (LineAhead)  // the last chunk prefetches its own blocks 14 and 15 again (in cache)
            hash_full_chunk_line_ahead(c, chunk, static_cast<uint32_t>(ctr), static_cast<uint32_t>(ctr >> 32), mode,
                                       kChunkEnd | (K == 1 ? root_flag : 0u), ea, oa,
                                       step + 1 < K ? ptr + static_cast<uint64_t>((k + 1) % K) * kChunkBytes
                                                    : chunk + (kBlocksPerChunk - 2) * kBlockBytes);
        else
            hash_full_chunk<Turns>(c, ptr + static_cast<uint64_t>(k) * kChunkBytes, static_cast<uint32_t>(ctr),
                            static_cast<uint32_t>(ctr >> 32), mode, kChunkEnd | (K == 1 ? root_flag : 0u));
        if (K == 1) return;
#pragma unroll
        for (int w = 0; w < 8; ++w) slots[(k * 8 + w) * kLanes] = c[w];
    }
    for (uint32_t width = K; width > 1; width /= 2) {
        for (uint32_t i = 0; i < width / 2; ++i) {
            uint32_t m[16];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                m[w] = slots[(2 * i * 8 + w) * kLanes];
                m[w + 8] = slots[((2 * i + 1) * 8 + w) * kLanes];
            }
#pragma unroll
            for (int w = 0; w < 8; ++w) c[w] = key[w];
            compress(c, m, 0, 0, kBlockBytes, mode | kParent | (width == 2 ? root_flag : 0u));
            if (width > 2) {
#pragma unroll
                for (int w = 0; w < 8; ++w) slots[(i * 8 + w) * kLanes] = c[w];
            }
        }
    }
}

// ---- full waves, staged loads (BLAKE3_GPU_STAGING=lds) ----------------------------------
// The same work as direct_subtree with the input staged through LDS. Each step stages 128
// bytes (two blocks) of every lane's current chunk in the wave's own 8 KiB of LDS:
// row r holds lane r's bytes, its 16-byte piece p at column p ^ (r & 7). The loads are
// direct-to-LDS and coalesced: load instruction j fills rows 8j..8j+7, lane i bringing
// piece (i & 7) ^ (i >> 3) of row 8j + (i >> 3), so every 128-byte line is fetched whole
// by 8 lanes of one instruction, and the XOR swizzle makes the lanes' row reads cover all
// LDS banks. The next step's loads are issued as soon as the current row is in
// registers, so they overlap two compressions.
constexpr uint32_t kStageBytes = kWaveLanes * 2 * kBlockBytes;  // 8 KiB per wave

// Rows of a wave whose runs of K chunks are evenly spaced (one message): row R starts at
// base + R * K KiB.
struct EvenRows {
    const uint8_t *lane_src;  // this lane's source within load 0
    uint64_t load_stride;     // 8 rows further per load instruction
    __device__ const uint8_t *ptr(uint32_t j) const { return lane_src + j * load_stride; }
};

// Rows at arbitrary addresses (batch): each lane keeps the sources of its 8 loads.
struct GatherRows {
    const uint8_t *src[8];
    __device__ const uint8_t *ptr(uint32_t j) const { return src[j]; }
};

__device__ __forceinline__ uint32_t stage_piece(uint32_t lw) { return (lw & 7u) ^ (lw >> 3); }

template <class Rows>
__device__ __forceinline__ void stage_issue(const Rows &rows, uint32_t off, uint32_t *stage) {
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(rows.ptr(j) + off),
                                         (__attribute__((address_space(3))) void *)(stage + j * 256), 16, 0, 0);
}

template <uint32_t K, class Rows>
__device__ __forceinline__ void staged_subtree(uint32_t (&c)[8], const Rows &rows, uint32_t *stage, uint64_t ctr0,
                                               const uint32_t (&key)[8], uint32_t mode, uint32_t root_flag) {
    const uint32_t lw = threadIdx.x % kWaveLanes;
    const uint4 *row = reinterpret_cast<const uint4 *>(stage) + lw * 8;
    uint32_t slot1c[8], slot2c[8];
    stage_issue(rows, 0, stage);
    for (uint32_t k = 0; k < K; ++k) {
#pragma unroll
        for (int w = 0; w < 8; ++w) c[w] = key[w];
        const uint64_t ctr = ctr0 + k;
        const uint32_t lo = static_cast<uint32_t>(ctr), hi = static_cast<uint32_t>(ctr >> 32);
        for (uint32_t bp = 0; bp < kBlocksPerChunk / 2; ++bp) {
            // this step's loads have landed in LDS: even block out of the lane's row
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            uint4 q0 = row[0 ^ (lw & 7u)], q1 = row[1 ^ (lw & 7u)], q2 = row[2 ^ (lw & 7u)], q3 = row[3 ^ (lw & 7u)];
            compress_block(c, Block{q0, q1, q2, q3}, lo, hi, mode | (bp == 0 ? kChunkStart : 0u));
            // odd block out, then refill the stage with the next step while it is compressed
            q0 = row[4 ^ (lw & 7u)];
            q1 = row[5 ^ (lw & 7u)];
            q2 = row[6 ^ (lw & 7u)];
            q3 = row[7 ^ (lw & 7u)];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (bp + 1 < kBlocksPerChunk / 2) stage_issue(rows, k * kChunkBytes + (bp + 1) * 2 * kBlockBytes, stage);
            else if (k + 1 < K) stage_issue(rows, (k + 1) * kChunkBytes, stage);
            compress_block(c, Block{q0, q1, q2, q3}, lo, hi,
                           mode | (bp + 1 == kBlocksPerChunk / 2 ? kChunkEnd | (K == 1 ? root_flag : 0u) : 0u));
        }
        if (K > 1) fold_chunk<K>(c, k, slot1c, slot2c, k + 1 < K, root_flag ? K - 1 : K, key, mode);
    }
}

__device__ __forceinline__ void store_digest(uint8_t *out, const uint32_t (&cv)[8]) {
#pragma unroll
    for (int w = 0; w < 8; ++w)
#pragma unroll
        for (int k = 0; k < 4; ++k) out[4 * w + k] = static_cast<uint8_t>(cv[w] >> (8 * k));
}

// Words j and 4 + j of a digest or CV (one lane of a quad's share of a node).
__device__ __forceinline__ void store_digest_pair(uint8_t *out, uint32_t j, uint32_t lo, uint32_t hi) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[4 * j + k] = static_cast<uint8_t>(lo >> (8 * k));
        out[16 + 4 * j + k] = static_cast<uint8_t>(hi >> (8 * k));
    }
}

__device__ __forceinline__ void store_cv_pair(uint32_t *dst, uint32_t j, uint32_t lo, uint32_t hi) {
    dst[j] = lo;
    dst[4 + j] = hi;
}

// Device-coherent forms for CVs another workgroup reads in the same launch (fused levels):
// agent-scope atomic stores and loads go to the coherence point the eight XCDs share,
// instead of an XCD's own L2.
__device__ __forceinline__ void store_word_coherent(uint32_t *dst, uint32_t v) {
    __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_word_coherent(const uint32_t *src) {
    return __hip_atomic_load(const_cast<uint32_t *>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Uniform batch: `segs` segments of `nodes` nodes each, segment s at lanes
// [s << lanes_log2, (s << lanes_log2) + nodes), all of one kind (whole messages, or one
// group of a message).
struct UniformSegs {
    uint32_t lanes_log2;
    uint32_t nodes;
    uint32_t segs;
    uint32_t first_msg;  // message of segment 0
    bool whole;          // segments are whole messages: their result goes to `digests`
    uint32_t top_flag;   // flag of a whole message's top compression: ROOT, or 0 for a subtree CV
    const uint32_t *keys;
    uint32_t key[8];
    uint32_t mode_flag;
    uint32_t *cv_out;
    uint64_t cv_slot;    // where a segment that is not a whole message writes its CV (cv_out + 8*cv_slot)
    bool coherent;       // that CV is read by another workgroup of this launch: device-coherent stores
    uint8_t *digests;

    __device__ uint32_t root_bit() const { return top_flag; }

    // node positions in use: the tree's levels fit the quad layout by this bound
    __device__ uint32_t used_positions() const { return segs << lanes_log2; }
    __device__ int seg_of(uint32_t pos) const {
        const uint32_t s = pos >> lanes_log2;
        return s < segs && pos - (s << lanes_log2) < nodes ? static_cast<int>(s) : -1;
    }
    __device__ uint32_t start(int s) const { return static_cast<uint32_t>(s) << lanes_log2; }
    __device__ uint32_t count(int) const { return nodes; }
    __device__ bool final(int) const { return whole; }
    __device__ uint32_t mode() const { return mode_flag; }
    __device__ void key_words(int s, uint32_t (&kw)[8]) const {
        if (keys) {
            load_cv(kw, keys + 8ull * (first_msg + static_cast<uint32_t>(s)));
        } else {
#pragma unroll
            for (int w = 0; w < 8; ++w) kw[w] = key[w];
        }
    }
    __device__ void emit(int s, const uint32_t (&cv)[8]) const {
        if (whole) {
            store_digest(digests + 32ull * (first_msg + static_cast<uint32_t>(s)), cv);
        } else if (coherent) {
#pragma unroll
            for (int w = 0; w < 8; ++w) store_word_coherent(cv_out + 8ull * cv_slot + w, cv[w]);
        } else {
            store_cv(cv_out + 8ull * cv_slot, cv);
        }
    }
    __device__ void emit_pair(int s, uint32_t j, uint32_t lo, uint32_t hi) const {
        if (whole) {
            store_digest_pair(digests + 32ull * (first_msg + static_cast<uint32_t>(s)), j, lo, hi);
        } else if (coherent) {
            store_word_coherent(cv_out + 8ull * cv_slot + j, lo);
            store_word_coherent(cv_out + 8ull * cv_slot + 4 + j, hi);
        } else {
            store_cv_pair(cv_out + 8ull * cv_slot, j, lo, hi);
        }
    }
};

// Batch: segments of this workgroup staged in LDS, plus the lane -> segment map.
struct BatchSegs {
    const Seg *seg;        // LDS
    const int *seg_of_pos; // LDS, one entry per lane position
    const uint32_t *keys;  // global, nullptr for default mode
    uint32_t *cv_out;
    uint8_t *digests;
    bool coherent;         // CVs are read by another workgroup of this launch: device-coherent stores
    const uint32_t *pos_info;  // LDS, per lane position: its segment's info word (stage_segments)
    const uint32_t *pos_key;   // LDS, per lane position: its segment's key, word w at w * kPosKeyStride

    __device__ uint32_t used_positions() const { return kLanes; }
    __device__ uint32_t root_bit() const { return kRoot; }
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
        if (final(s)) {
            store_digest(digests + 32ull * seg[s].msg, cv);
        } else if (coherent) {
#pragma unroll
            for (int w = 0; w < 8; ++w) store_word_coherent(cv_out + 8ull * seg[s].dst + w, cv[w]);
        } else {
            store_cv(cv_out + 8ull * seg[s].dst, cv);
        }
    }
    __device__ void emit_pair(int s, uint32_t j, uint32_t lo, uint32_t hi) const {
        if (final(s)) {
            store_digest_pair(digests + 32ull * seg[s].msg, j, lo, hi);
        } else if (coherent) {
            store_word_coherent(cv_out + 8ull * seg[s].dst + j, lo);
            store_word_coherent(cv_out + 8ull * seg[s].dst + 4 + j, hi);
        } else {
            store_cv_pair(cv_out + 8ull * seg[s].dst, j, lo, hi);
        }
    }
};

// Loads this workgroup's segments into LDS and maps every lane position to its segment
// (or -1) and to that segment's info word, so that a tree level reads both at once rather
// than one after the other. Segments are sorted by lane start.
template <uint32_t C>
__device__ __forceinline__ void stage_segments(const uint32_t *wg_first_seg, const Seg *segs, Seg *s_seg,
                                               int *s_seg_of, uint32_t *s_pos_info) {
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
    s_pos_info[lane] = s >= 0 ? s_seg[s].info : 0u;
    __syncthreads();
}

// ---- a tree node position's segment ---------------------------------------------------

// The segment of a node position as the tree levels use it: its index (-1: no segment),
// first position and node count, and whether its result is a message's digest.
struct NodeRef {
    int s;
    uint32_t start, n;
    bool fin;
};

// Stride, in words, of a per-position key table (word w of position x at
// w * kPosKeyStride + x): one word of padding spreads the eight words over LDS banks.
constexpr uint32_t kPosKeyStride = kLanes + 1;
constexpr uint32_t kPosKeyWords = 8 * kPosKeyStride;

// Generic forms, from the Segs type's own lookups.
template <class Segs>
__device__ __forceinline__ NodeRef seg_node(const Segs &sg, uint32_t pos) {
    const int s = sg.seg_of(pos);
    if (s < 0) return NodeRef{-1, 0u, 0u, false};
    return NodeRef{s, sg.start(s), sg.count(s), sg.final(s)};
}
template <class Segs>
__device__ __forceinline__ void seg_key_words(const Segs &sg, const NodeRef &nd, uint32_t, uint32_t (&kw)[8]) {
    sg.key_words(nd.s < 0 ? 0 : nd.s, kw);
}

// Batch segments: both lookups read the position tables, with no read waiting for another.
__device__ __forceinline__ NodeRef seg_node(const BatchSegs &sg, uint32_t pos) {
    const int s = sg.seg_of_pos[pos];
    const uint32_t info = sg.pos_info[pos];
    return NodeRef{s, seg_lane(info), seg_count(info), seg_final(info)};
}
__device__ __forceinline__ void seg_key_words(const BatchSegs &sg, const NodeRef &, uint32_t pos,
                                              uint32_t (&kw)[8]) {
    if (sg.keys) {
#pragma unroll
        for (int w = 0; w < 8; ++w) kw[w] = sg.pos_key[w * kPosKeyStride + pos];
    } else {
#pragma unroll
        for (int w = 0; w < 8; ++w) kw[w] = kIV[w];
    }
}

// Words j and 4 + j of the key of the segment at pos (a quad lane's share).
template <class Segs>
__device__ __forceinline__ void seg_key_pair(const Segs &sg, const NodeRef &nd, uint32_t pos, uint32_t j,
                                             uint32_t &lo, uint32_t &hi) {
    uint32_t kw[8];
    seg_key_words(sg, nd, pos, kw);
    lo = pick4(kw[0], kw[1], kw[2], kw[3], j);
    hi = pick4(kw[4], kw[5], kw[6], kw[7], j);
}
__device__ __forceinline__ void seg_key_pair(const BatchSegs &sg, const NodeRef &, uint32_t pos, uint32_t j,
                                             uint32_t &lo, uint32_t &hi) {
    if (sg.keys) {
        lo = sg.pos_key[j * kPosKeyStride + pos];
        hi = sg.pos_key[(4 + j) * kPosKeyStride + pos];
    } else {
        lo = pick4(kIV[0], kIV[1], kIV[2], kIV[3], j);
        hi = pick4(kIV[4], kIV[5], kIV[6], kIV[7], j);
    }
}

// compress_quad with this lane's message words read from LDS (src[moff[4r + t]] is its
// t-th word of round r). The words of the first four rounds are read at once and those of
// round r + 4 while round r runs (at most 16 reads in flight), so that no round waits for
// LDS after the first; the compiler barrier keeps the reads in that order. The same in two
// parts, quad_msg_head and compress_quad_lds_rest, lets a caller issue the first reads
// before other LDS reads that it waits for first. (compress_quad_lds stays one piece: the
// compiler schedules its callers' chunk loops better that way, measured.)
__device__ __forceinline__ void quad_msg_head(uint32_t (&m)[28], const uint32_t *src, const uint32_t (&moff)[28]) {
#pragma unroll
    for (int t = 0; t < 16; ++t) m[t] = src[moff[t]];
}
__device__ __forceinline__ void compress_quad_lds_rest(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d,
                                                       uint32_t (&m)[28], const uint32_t *src,
                                                       const uint32_t (&moff)[28]) {
#pragma unroll
    for (int r = 0; r < 7; ++r) {
        if (r + 4 < 7) {
#pragma unroll
            for (int t = 0; t < 4; ++t) m[4 * (r + 4) + t] = src[moff[4 * (r + 4) + t]];
        }
        asm volatile("" ::: "memory");
        quad_round_words(a, b, c, d, m[4 * r], m[4 * r + 1], m[4 * r + 2], m[4 * r + 3]);
    }
}
__device__ __forceinline__ void compress_quad_lds(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d,
                                                  const uint32_t *src, const uint32_t (&moff)[28]) {
    uint32_t m[28];
#pragma unroll
    for (int t = 0; t < 16; ++t) m[t] = src[moff[t]];
#pragma unroll
    for (int r = 0; r < 7; ++r) {
        if (r + 4 < 7) {
#pragma unroll
            for (int t = 0; t < 4; ++t) m[4 * (r + 4) + t] = src[moff[4 * (r + 4) + t]];
        }
        asm volatile("" ::: "memory");
        quad_round_words(a, b, c, d, m[4 * r], m[4 * r + 1], m[4 * r + 2], m[4 * r + 3]);
    }
}

// Output nodes per level up to which a level runs on quads (four lanes per node): at
// most 64 nodes would fill one wave or less at one lane per node, where on quads they
// fill up to four waves (one per SIMD of a 256-lane workgroup) and each node's
// compression has a quarter of the dependent chain.
constexpr uint32_t kQuadLevelNodes = 64;

// Levels l of a tree over `used` node positions with more than kQuadLevelNodes output
// positions (these run one lane per node).
__device__ __forceinline__ uint32_t lane_levels(uint32_t used) {
    uint32_t l = 0;
    while (((used - 1) >> (l + 1)) + 1 > kQuadLevelNodes) ++l;
    return l;
}

// Segment kinds whose lookups are LDS reads (batch tables): their tree levels issue the
// lookups, the key reads and the first message reads before waiting for any of them. The
// others compute their lookups, and keep the order in which the compiler schedules them
// best (measured: issuing the reads first there cost 2-3% at 1-4 MiB).
template <class Segs>
struct EarlyLevelReads : std::false_type {};
template <>
struct EarlyLevelReads<BatchSegs> : std::true_type {};

// One level of tree_levels_quad for segment kinds whose lookups are computed: level l's
// nodes are read from buffer Src (a compile-time index, so that every message read is one LDS instruction with a constant
// offset) and level l + 1's written to the other buffer.
template <uint32_t C, uint32_t Src, class Segs>
__device__ __forceinline__ void quad_level_computed(const Segs &sg, uint32_t l, uint32_t p, uint32_t j,
                                           const uint32_t (&moff)[28], uint32_t (*buf)[8][C]) {
    const uint32_t pos = p << (l + 1);
    if (pos >= C) return;
    const int s = sg.seg_of(pos);
    if (s < 0) return;
    const uint32_t start = sg.start(s), n = sg.count(s), r = ceil_log2(n);
    if (l >= r) return;  // segment already reduced to one node
    // every condition above depends on p only: the quad's four lanes stay together
    const uint32_t *src = &buf[Src][0][0];
    uint32_t lo, hi;
    if ((((2 * p + 1) << l) - start) < n) {  // a right child exists
        uint32_t kw[8];
        sg.key_words(s, kw);
        uint32_t a = pick4(kw[0], kw[1], kw[2], kw[3], j);
        uint32_t b = pick4(kw[4], kw[5], kw[6], kw[7], j);
        uint32_t c = pick4(kIV[0], kIV[1], kIV[2], kIV[3], j);
        const uint32_t flags = sg.mode() | kParent | (sg.final(s) && l + 1 == r ? sg.root_bit() : 0u);
        uint32_t d = j == 3u ? flags : (j == 2u ? kBlockBytes : 0u);  // counter 0, length 64
        compress_quad_lds(a, b, c, d, src, moff);
        lo = a ^ c;
        hi = b ^ d;
    } else {  // carry node 2p up unchanged
        lo = src[j * C + 2 * p];
        hi = src[(4 + j) * C + 2 * p];
    }
    uint32_t *dst = &buf[1 - Src][0][0];
    dst[j * C + p] = lo;
    dst[(4 + j) * C + p] = hi;
    if (l + 1 == r) sg.emit_pair(s, j, lo, hi);
}

// One level of tree_levels_quad for the batch segment kinds: the same, with the node's
// segment, its key words and the first sixteen message words read before any of them is
// waited for.
template <uint32_t C, uint32_t Src, class Segs>
__device__ __forceinline__ void quad_level_early(const Segs &sg, uint32_t l, uint32_t p, uint32_t j,
                                                 const uint32_t (&moff)[28], uint32_t (*buf)[8][C]) {
    const uint32_t pos = p << (l + 1);
    if (pos >= C) return;  // so p < C / 2: every message offset lies inside the level buffer
    const uint32_t *src = &buf[Src][0][0];
    const NodeRef nd = seg_node(sg, pos);
    uint32_t m[28];
    quad_msg_head(m, src, moff);
    uint32_t klo, khi;
    seg_key_pair(sg, nd, pos, j, klo, khi);
    if (nd.s < 0) return;
    const uint32_t r = ceil_log2(nd.n);
    if (l >= r) return;  // segment already reduced to one node
    // every condition above depends on p only: the quad's four lanes stay together
    uint32_t lo, hi;
    if ((((2 * p + 1) << l) - nd.start) < nd.n) {  // a right child exists
        uint32_t a = klo, b = khi;
        uint32_t c = pick4(kIV[0], kIV[1], kIV[2], kIV[3], j);
        const uint32_t flags = sg.mode() | kParent | (nd.fin && l + 1 == r ? sg.root_bit() : 0u);
        uint32_t d = j == 3u ? flags : (j == 2u ? kBlockBytes : 0u);  // counter 0, length 64
        compress_quad_lds_rest(a, b, c, d, m, src, moff);
        lo = a ^ c;
        hi = b ^ d;
    } else {  // carry node 2p up unchanged
        lo = src[j * C + 2 * p];
        hi = src[(4 + j) * C + 2 * p];
    }
    uint32_t *dst = &buf[1 - Src][0][0];
    dst[j * C + p] = lo;
    dst[(4 + j) * C + p] = hi;
    if (l + 1 == r) sg.emit_pair(nd.s, j, lo, hi);
}

template <uint32_t C, uint32_t Src, class Segs>
__device__ __forceinline__ void quad_level(const Segs &sg, uint32_t l, uint32_t p, uint32_t j,
                                           const uint32_t (&moff)[28], uint32_t (*buf)[8][C]) {
    if constexpr (EarlyLevelReads<Segs>::value) quad_level_early<C, Src>(sg, l, p, j, moff, buf);
    else quad_level_computed<C, Src>(sg, l, p, j, moff, buf);
}

// Levels l .. levels-1 of the tree on quads, the level-l nodes being in buf[l & 1]
// (word w of node x at buf[.][w][x]). Output node p is the parent of nodes 2p and 2p+1,
// whose 16 words are the message (left node's words 0..7, then the right node's), and
// runs on lanes 4p..4p+3, lane j holding words j and 4 + j of it; moff holds the word
// offsets, within a level buffer, of the 28 words this lane reads. A level over n nodes
// takes 2n lanes (four per output node); lane_levels leaves to the quads only levels with
// at most kQuadLevelNodes output nodes. The loop is unrolled by two so that each copy of
// a level reads a fixed buffer.
// InLoop: the caller runs this inside a loop; the lane's offsets are then made opaque to
// the optimiser so that they are computed here rather than hoisted out of that loop,
// where they would hold 28 registers across the rest of the kernel.
template <uint32_t C, class Segs, bool InLoop = false>
__device__ __forceinline__ void tree_levels_quad(const Segs &sg, uint32_t l, uint32_t levels,
                                                 uint32_t (*buf)[8][C]) {
    const uint32_t lane = threadIdx.x;
    uint32_t p = lane >> 2, j = lane & 3u;
    if (InLoop) asm volatile("" : "+v"(p), "+v"(j));
    uint32_t moff[28];
#pragma unroll
    for (int r = 0; r < 7; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t idx = (static_cast<uint32_t>(kQuadWord.at[r][t]) >> (4 * j)) & 15u;
            moff[4 * r + t] = (idx & 7u) * C + 2 * p + (idx >> 3);
        }
    if (l < levels && (l & 1u)) {
        __syncthreads();
        quad_level<C, 1>(sg, l, p, j, moff, buf);
        ++l;
    }
    for (; l < levels; l += 2) {
        __syncthreads();
        quad_level<C, 0>(sg, l, p, j, moff, buf);
        if (l + 1 == levels) break;
        __syncthreads();
        quad_level<C, 1>(sg, l + 1, p, j, moff, buf);
    }
}

// The fused partial Merkle reduction. On entry lane x holds the level-0 node x in `cv`
// (if it belongs to a segment). Each segment's result is emitted by the lane (or quad)
// that computes it, at the level where the segment reaches a single node. Levels with
// more than kQuadLevelNodes output positions run one lane per node; the sparse top of
// the tree runs one quad per node, output node p on lanes 4p..4p+3.
template <uint32_t C, class Segs, bool InLoop = false>
__device__ __forceinline__ void tree_reduce(const uint32_t (&cv)[8], const Segs &sg, uint32_t levels,
                                            uint32_t (*buf)[8][C]) {
    const uint32_t lane = threadIdx.x;
    const int s0 = sg.seg_of(lane);
    if (s0 >= 0) {
#pragma unroll
        for (int w = 0; w < 8; ++w) buf[0][w][lane] = cv[w];
        if (sg.count(s0) == 1) sg.emit(s0, cv);
    }
    const uint32_t lane_lv = lane_levels(sg.used_positions());
    uint32_t l = 0;
    if constexpr (EarlyLevelReads<Segs>::value) {
        for (; l < levels && l < lane_lv; ++l) {
            __syncthreads();
            const uint32_t pos = lane << (l + 1);  // first leaf position under output node `lane`
            if (pos >= C) continue;                // so lane < C / 2: both children lie in the buffer
            // the segment, the children and the key are read before any of them is waited for
            const NodeRef nd = seg_node(sg, pos);
            const uint32_t(*src)[C] = buf[l & 1];
            uint32_t m[16];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const uint2 pr = *reinterpret_cast<const uint2 *>(&src[w][2 * lane]);
                m[w] = pr.x;
                m[w + 8] = pr.y;
            }
            uint32_t node[8];
            seg_key_words(sg, nd, pos, node);
            if (nd.s < 0) continue;
            const uint32_t r = ceil_log2(nd.n);
            if (l >= r) continue;  // segment already reduced to one node
            if ((((2 * lane + 1) << l) - nd.start) < nd.n) {  // a right child exists
                const uint32_t flags = sg.mode() | kParent | (nd.fin && l + 1 == r ? sg.root_bit() : 0u);
                compress(node, m, 0, 0, kBlockBytes, flags);
            } else {  // carry the left child up unchanged
#pragma unroll
                for (int w = 0; w < 8; ++w) node[w] = m[w];
            }
#pragma unroll
            for (int w = 0; w < 8; ++w) buf[(l + 1) & 1][w][lane] = node[w];
            if (l + 1 == r) sg.emit(nd.s, node);
        }
    } else {
        for (; l < levels && l < lane_lv; ++l) {
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
                const uint32_t flags = sg.mode() | kParent | (sg.final(s) && l + 1 == r ? sg.root_bit() : 0u);
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
    if (l < levels) tree_levels_quad<C, Segs, InLoop>(sg, l, levels, buf);
}

// ---- kernels ---------------------------------------------------------------------------

// LDS of the leaf kernel: during the chunk phase the waves' stage buffers (staged
// loads) or the lanes' chunk slots (direct loads); then the tree's two level buffers (a
// barrier separates the two uses).
template <uint32_t K, bool Staged>
constexpr uint32_t leaf_lds_words() {
    constexpr uint32_t tree = 2 * 8 * kLanes;
    constexpr uint32_t chunk_phase = Staged ? (kLanes / kWaveLanes) * kStageBytes / 4 : (K > 1 ? K * 8 * kLanes : 0);
    return tree > chunk_phase ? tree : chunk_phase;
}

// Sets the fields of a UniformSegs that do not depend on the pass.
template <typename Args>
__device__ __forceinline__ void uniform_common(UniformSegs &sg, const Args &a, uint32_t block) {
    sg.top_flag = a.root_flag;
    sg.keys = a.keys;
#pragma unroll
    for (int w = 0; w < 8; ++w) sg.key[w] = a.key[w];
    sg.mode_flag = a.mode;
    sg.cv_out = a.cv_out;
    sg.cv_slot = block;
    sg.coherent = false;
    sg.digests = a.digests;
}

// Fused level passes (UniformLeafArgs::levels): called by the whole workgroup after its
// leaf tree has written group CV blockIdx.x with device-coherent stores. Each wave waits
// for its stores to complete, a barrier, then one agent-scope atomic ticket per
// workgroup; the last arrival of a group reads the group's CVs with device-coherent loads,
// sets the ticket back to zero (so tickets need no clearing between launches: every
// launch leaves them as it found them) and reduces the CVs with the tree of the level
// kernel, on quads up to the group's own size.
// Ordering: the CV words are only ever accessed as agent-scope atomics, which gfx950
// performs at the point of coherence shared by the XCDs (the compiler emits them as sc1
// stores and loads). A writer's ticket is issued only after vmcnt(0) has seen its CV
// stores complete there, and the last arrival issues its CV loads only after its ticket
// has returned (the outcome reaches the other waves through LDS and a barrier), so those
// loads find every CV of the group. The release/acquire form (an acquire-release ticket,
// which adds an L2 write-back before it and an invalidation after it) gives the same
// digests and measured 0.5-27% slower.
// LDS words fused_levels needs at `lds`: the level tree's two buffers of 8 x 256 words.
constexpr uint32_t kFusedLevelLdsWords = 2 * 8 * kLevelLanes;

__device__ void fused_levels(const UniformLeafArgs &a, uint32_t *lds) {
    const uint32_t lane = threadIdx.x;
    auto buf = reinterpret_cast<uint32_t(*)[8][kLevelLanes]>(lds);
    const uint32_t msg = blockIdx.x / a.groups;
    uint64_t idx = blockIdx.x - static_cast<uint64_t>(msg) * a.groups;  // this node at level L
    for (uint32_t L = 0; L < a.levels; ++L) {
        const uint64_t g_in = a.lvl_g[L], g_out = a.lvl_g[L + 1];
        const uint64_t group = idx / kLevelLanes, first = group * kLevelLanes;
        const uint32_t count = g_in - first < kLevelLanes ? static_cast<uint32_t>(g_in - first) : kLevelLanes;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's CV stores have completed
        __syncthreads();  // ... in every wave; the tree is done with the LDS: word 0 carries the outcome
        if (lane == 0) {
            uint32_t *ticket = a.lvl_ctr[L] + msg * g_out + group;
            const bool last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == count;
            if (last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            lds[0] = last ? 1u : 0u;
        }
        __syncthreads();
        const bool last = lds[0] != 0;
        __syncthreads();  // everyone has read it before the tree writes over it
        if (!last) return;
        uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (lane < count) {
            const uint32_t *src = a.lvl_cv[L] + 8 * (msg * g_in + first + lane);
#pragma unroll
            for (int w = 0; w < 8; ++w) cv[w] = load_word_coherent(src + w);
        }
        UniformSegs sg{};
        uniform_common(sg, a, blockIdx.x);
        sg.lanes_log2 = ceil_log2(count);  // the group's nodes at positions 0 .. count - 1
        sg.nodes = count;
        sg.segs = 1;
        sg.first_msg = msg;
        sg.whole = g_out == 1;
        sg.cv_out = L + 1 < a.levels ? a.lvl_cv[L + 1] : nullptr;
        sg.cv_slot = msg * g_out + group;
        sg.coherent = true;
        tree_reduce<kLevelLanes, UniformSegs, true>(cv, sg, ceil_log2(count), buf);
        idx = group;
    }
}

// Case A groups: `per_wg` messages per workgroup, R = 1 << lanes_log2 lanes each.
__device__ __forceinline__ void uniform_case_a(UniformSegs &sg, uint32_t lanes_per_msg, uint32_t n_msgs,
                                               uint32_t wg_lanes, uint32_t block) {
    sg.lanes_log2 = static_cast<uint32_t>(__builtin_ctz(lanes_per_msg));
    const uint32_t per_wg = wg_lanes >> sg.lanes_log2;
    sg.first_msg = block * per_wg;
    sg.segs = n_msgs - sg.first_msg < per_wg ? n_msgs - sg.first_msg : per_wg;
}

// One workgroup of the lane-per-chunk leaf: workgroup `block` of the grid that `a`
// describes, with leaf_lds_words<K, Staged>() words of LDS at `lds`. Fused: the level
// passes run in this launch (fused_levels, and `block` is then the launch's own workgroup
// index); a separate instantiation, so that the registers the level tree needs do not
// weigh on the default leaf.
template <uint32_t K, bool Staged, bool Fused>
__device__ __forceinline__ void leaf_uniform_wg(const UniformLeafArgs &a, uint32_t block, uint32_t *lds) {
    const uint32_t lane = threadIdx.x;
    constexpr uint64_t kWgChunks = static_cast<uint64_t>(kLanes) * K;
    UniformSegs sg{};
    uint64_t first_chunk = 0;
    if (a.lanes_per_msg != 0) {  // case A: whole messages, several per workgroup
        uniform_case_a(sg, a.lanes_per_msg, a.n_msgs, kLanes, block);
        sg.nodes = static_cast<uint32_t>((a.n_chunks + K - 1) / K);
        sg.whole = a.may_root != 0;
    } else {  // case B: one group of one message
        sg.lanes_log2 = 8;
        sg.first_msg = block / a.groups;
        sg.segs = 1;
        first_chunk = static_cast<uint64_t>(block - sg.first_msg * a.groups) * kWgChunks;
        const uint64_t left = a.n_chunks - first_chunk;
        sg.nodes = left >= kWgChunks ? kLanes : static_cast<uint32_t>((left + K - 1) / K);
        sg.whole = a.may_root != 0 && a.groups == 1;
    }
    uniform_common(sg, a, block);
    sg.coherent = Fused;  // group CVs are read by the fused levels

    const uint32_t s = lane >> sg.lanes_log2, x = lane - (s << sg.lanes_log2);
    uint32_t nl = 0, last_len = kChunkBytes;
    uint64_t c0 = 0;
    const uint8_t *ptr = a.base;
    uint32_t key[8];
    sg.key_words(s < sg.segs ? static_cast<int>(s) : 0, key);
    if (s < sg.segs && x < sg.nodes) {
        c0 = first_chunk + static_cast<uint64_t>(x) * K;
        nl = a.n_chunks - c0 < K ? static_cast<uint32_t>(a.n_chunks - c0) : K;
        const uint64_t rem = a.len - (c0 + nl - 1) * kChunkBytes;  // bytes from the lane's last chunk on
        last_len = a.len == 0 ? 0u : (rem < kChunkBytes ? static_cast<uint32_t>(rem) : kChunkBytes);
        ptr = a.base + static_cast<uint64_t>(sg.first_msg + s) * a.stride + c0 * kChunkBytes;
    }
    // a message of one node: the lane's own subtree is the whole tree
    const uint32_t root_flag = sg.whole && sg.nodes == 1 ? sg.top_flag : 0u;
    uint32_t cv[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) cv[w] = key[w];
    if (__ballot(nl != K || last_len != kChunkBytes) == 0) {
        if (Staged) {
            const uint32_t lw = lane % kWaveLanes;
            uint32_t *stage = lds + (lane / kWaveLanes) * (kStageBytes / 4);
            if (a.lanes_per_msg == 0) {  // the wave's runs of K chunks are evenly spaced
                // lane lw reads from ptr - (lw - (lw >> 3)) * K chunks: row lw >> 3 of load 0
                const EvenRows rows{ptr - static_cast<uint64_t>(lw - (lw >> 3)) * K * kChunkBytes +
                                        16 * stage_piece(lw),
                                    8ull * K * kChunkBytes};
                staged_subtree<K>(cv, rows, stage, a.chunk_base + c0, key, a.mode, root_flag);
            } else {  // gather the 8 rows each lane loads for
                const uint64_t my = reinterpret_cast<uint64_t>(ptr);
                GatherRows rows;
#pragma unroll
                for (uint32_t j = 0; j < 8; ++j)
                    rows.src[j] = reinterpret_cast<const uint8_t *>(__shfl(my, static_cast<int>(8 * j + (lw >> 3)))) +
                                  16 * stage_piece(lw);
                staged_subtree<K>(cv, rows, stage, a.chunk_base + c0, key, a.mode, root_flag);
            }
        } else {
            direct_subtree<K, true>(cv, ptr, a.chunk_base + c0, key, a.mode, root_flag, lds + lane);
        }
    } else if (nl > 0) {
        lane_subtree<K>(cv, ptr, nl, last_len, a.chunk_base + c0, key, a.mode, root_flag != 0);
    }
    __syncthreads();  // every wave is done with its stage buffer or slots before the tree reuses them
    tree_reduce<kLanes>(cv, sg, ceil_log2(sg.nodes), reinterpret_cast<uint32_t(*)[8][kLanes]>(lds));
    if (Fused) fused_levels(a, lds);
}

template <uint32_t K, bool Staged, bool Fused>
__global__ __launch_bounds__(kLeafLanes) void leaf_uniform_kernel(UniformLeafArgs a) {
    static_assert(!Fused || leaf_lds_words<K, Staged>() >= kFusedLevelLdsWords, "the fused levels fit the LDS");
    __shared__ __attribute__((aligned(16))) uint32_t lds[leaf_lds_words<K, Staged>()];
    leaf_uniform_wg<K, Staged, Fused>(a, blockIdx.x, lds);
}

__global__ __launch_bounds__(kLevelLanes) void level_uniform_kernel(UniformLevelArgs a) {
    __shared__ uint32_t buf[2][8][kLevelLanes];
    const uint32_t lane = threadIdx.x;
    UniformSegs sg{};
    uint64_t first_cv = 0;
    if (a.lanes_per_msg != 0) {  // case A: the last g_in CVs of several messages, finished here
        uniform_case_a(sg, a.lanes_per_msg, a.n_msgs, kLevelLanes, blockIdx.x);
        sg.nodes = static_cast<uint32_t>(a.g_in);
        sg.whole = true;
    } else {  // case B: 256 CVs (or the rest) of one message
        sg.lanes_log2 = 8;
        sg.first_msg = blockIdx.x / a.g_out;
        sg.segs = 1;
        first_cv = static_cast<uint64_t>(blockIdx.x - sg.first_msg * a.g_out) * kLevelLanes;
        const uint64_t left = a.g_in - first_cv;
        sg.nodes = left < kLevelLanes ? static_cast<uint32_t>(left) : kLevelLanes;
        sg.whole = false;
    }
    uniform_common(sg, a, blockIdx.x);
    const uint32_t s = lane >> sg.lanes_log2, x = lane - (s << sg.lanes_log2);
    uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (s < sg.segs && x < sg.nodes)
        load_cv(cv, a.cv_in + 8 * (static_cast<uint64_t>(sg.first_msg + s) * a.g_in + first_cv + x));
    tree_reduce<kLevelLanes>(cv, sg, ceil_log2(sg.nodes), buf);
}

// ---- small inputs: one quad per chunk -------------------------------------------------
// With a few thousand chunks the lane-per-chunk leaf cannot fill the chip, and its time
// is the latency of 16 sequential compressions on one lane plus the tree. Here a quad
// hashes each chunk (compress_quad, a third of the latency): a workgroup of 256 lanes
// takes kQuadLeafChunks = 64 chunks, loads them whole (16-byte loads, zero past the end of
// a short chunk) and stages each block in LDS as its compression comes, runs their blocks,
// and reduces the chunk CVs on quads.

// f(std::integral_constant<uint32_t, b>) for the blocks b = 0..15 of a chunk, in order: one
// copy of f's body per block, each with its block index a compile-time constant.
template <class F, uint32_t... Bs>
__device__ __forceinline__ void for_each_block_of(F &&f, std::integer_sequence<uint32_t, Bs...>) {
    (f(std::integral_constant<uint32_t, Bs>{}), ...);
}
template <class F>
__device__ __forceinline__ void for_each_block(F &&f) {
    for_each_block_of(f, std::make_integer_sequence<uint32_t, kBlocksPerChunk>{});
}

// Words per staged chunk row in LDS: a ring of two blocks (block b in slot b & 1; a slot is
// written again two blocks later, after the quad's reads of it, which its wave performs in
// order) plus 4 words of padding. Rows a multiple of 32 words apart would put the same word
// of every quad's chunk in one bank, and each message read of the compression (four words
// per lane per round, a different quad per chunk) would be an 8-way bank conflict per
// half-wave; with rows 4 banks apart it averages 1.8-way (3 at worst), the 64 lanes of a wave
// spread over the 32 banks.
constexpr uint32_t kQuadRowWords = 2 * kBlockBytes / 4 + 4;

// LDS of the quad leaf: the staged blocks (9 KiB); afterwards the tree's level buffers (4 KiB).
constexpr uint32_t kQuadLeafLdsWords = kQuadLeafChunks * kQuadRowWords;
static_assert(kQuadLeafLdsWords >= 2 * 8 * kQuadLeafChunks, "the tree's level buffers fit the staging rows");

// One workgroup of the quad leaf: workgroup `block` of the grid that `a` describes, with
// kQuadLeafLdsWords words of LDS at `lds` (Fused: `block` is the launch's own workgroup index).
template <bool Fused>
__device__ __forceinline__ void leaf_quad_wg(const UniformLeafArgs &a, uint32_t block, uint32_t *lds) {
    const uint32_t lane = threadIdx.x, q = lane >> 2, j = lane & 3u;
    UniformSegs sg{};
    uint64_t first_chunk = 0;
    if (a.lanes_per_msg != 0) {  // case A: whole messages, R chunk slots each
        uniform_case_a(sg, a.lanes_per_msg, a.n_msgs, kQuadLeafChunks, block);
        sg.nodes = static_cast<uint32_t>(a.n_chunks);
        sg.whole = a.may_root != 0;
    } else {  // case B: 64 chunks (or the rest) of one message
        sg.lanes_log2 = 6;
        sg.first_msg = block / a.groups;
        sg.segs = 1;
        first_chunk = static_cast<uint64_t>(block - sg.first_msg * a.groups) * kQuadLeafChunks;
        const uint64_t left = a.n_chunks - first_chunk;
        sg.nodes = left >= kQuadLeafChunks ? kQuadLeafChunks : static_cast<uint32_t>(left);
        sg.whole = a.may_root != 0 && a.groups == 1;
    }
    uniform_common(sg, a, block);
    sg.coherent = Fused;  // group CVs are read by the fused levels

    // chunk slot q of the workgroup: chunk x of segment s
    const uint32_t s = q >> sg.lanes_log2, x = q - (s << sg.lanes_log2);
    const bool active = s < sg.segs && x < sg.nodes;  // the same for the quad's 4 lanes
    uint32_t *mine = lds + q * kQuadRowWords;
    uint32_t lo = 0, hi = 0;  // this lane's CV words j and 4 + j
    uint32_t clen = 0;
    uint4 piece[kBlocksPerChunk];  // lane j's 16-byte piece j of every block of the quad's chunk
    uint4 tail = make_uint4(0, 0, 0, 0);
    uint32_t tail_at = kChunkBytes;  // byte offset of the chunk's partly valid piece, if any
    uint32_t kw[8];
    if (active) {
        // the key first: loads complete in issue order, so waiting for a per-message key
        // loaded after the chunk would wait for the whole chunk
        sg.key_words(static_cast<int>(s), kw);
        const uint64_t ci = first_chunk + x;
        const uint8_t *chunk = a.base + static_cast<uint64_t>(sg.first_msg + s) * a.stride + ci * kChunkBytes;
        const uint64_t rem = a.len - ci * kChunkBytes;
        clen = a.len == 0 ? 0u : (rem < kChunkBytes ? static_cast<uint32_t>(rem) : kChunkBytes);
        // all sixteen loads are issued here, one 16-byte load each with no branch (a piece not
        // wholly inside the chunk's bytes comes from the zero piece), so that the wait before
        // block b is for the loads of blocks 0..b only (loads complete in issue order); each
        // block's pieces go to LDS just before the quad compresses that block
#pragma unroll
        for (uint32_t i = 0; i < kBlocksPerChunk; ++i) piece[i] = load_piece_or_zero(chunk, 64 * i + 16 * j, clen);
        if (clen & 15u) {  // the piece holding the last byte, read byte by byte by its lane
            tail_at = clen & ~15u;
            if (((tail_at >> 4) & 3u) == j) tail = load_tail_piece(chunk, clen);
        }
    }
    if (active) {
        uint32_t moff[28];  // block word offsets of this lane's 28 message words
#pragma unroll
        for (int r = 0; r < 7; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t) moff[4 * r + t] = (static_cast<uint32_t>(kQuadWord.at[r][t]) >> (4 * j)) & 15u;
        lo = pick4(kw[0], kw[1], kw[2], kw[3], j);
        hi = pick4(kw[4], kw[5], kw[6], kw[7], j);
        const uint64_t ctr = a.chunk_base + first_chunk + x;
        const uint32_t nb = clen == 0 ? 1u : (clen + kBlockBytes - 1) / kBlockBytes;
        const uint32_t end_flags = kChunkEnd | (sg.whole && sg.nodes == 1 ? sg.top_flag : 0u);
        const uint32_t iv_j = pick4(kIV[0], kIV[1], kIV[2], kIV[3], j);
        // one copy per block (a compile-time block index): the pieces stay in registers and
        // every message read has a constant offset from the lane's precomputed addresses
        for_each_block([&](auto bc) __attribute__((always_inline)) {
            constexpr uint32_t b = decltype(bc)::value;
            if (b < nb) {  // nb is the same for the quad's four lanes
                // the partly valid piece replaces the zeros loaded for it (a second store by the
                // same lane, so that the array is only ever indexed by constants)
                reinterpret_cast<uint4 *>(mine)[4 * (b & 1) + j] = piece[b];
                if (tail_at == 64 * b + 16 * j) reinterpret_cast<uint4 *>(mine)[4 * (b & 1) + j] = tail;
                // the quad reads what its own lanes wrote (same wave, LDS in order): keep
                // the compiler from moving the reads above the writes
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
                const uint32_t last = b + 1 == nb;
                const uint32_t flags = sg.mode() | (b == 0 ? kChunkStart : 0u) | (last ? end_flags : 0u);
                const uint32_t blen = last ? clen - kBlockBytes * b : kBlockBytes;
                uint32_t va = lo, vb = hi, vc = iv_j;
                uint32_t vd = pick4(static_cast<uint32_t>(ctr), static_cast<uint32_t>(ctr >> 32), blen, flags, j);
                compress_quad_lds(va, vb, vc, vd, mine + 16 * (b & 1), moff);
                lo = va ^ vc;
                hi = vb ^ vd;
            }
        });
    }
    __syncthreads();  // every quad is done with its staged chunk: the tree reuses the LDS
    auto buf = reinterpret_cast<uint32_t(*)[8][kQuadLeafChunks]>(lds);
    if (active) {
        buf[0][j][q] = lo;
        buf[0][4 + j][q] = hi;
        if (sg.nodes == 1) sg.emit_pair(static_cast<int>(s), j, lo, hi);
    }
    tree_levels_quad<kQuadLeafChunks>(sg, 0, ceil_log2(sg.nodes), buf);
    if (Fused) fused_levels(a, lds);
}

template <bool Fused>
__global__ __launch_bounds__(kLeafLanes) void leaf_quad_kernel(UniformLeafArgs a) {
    // the fused levels' buffers are larger than the staged blocks
    constexpr uint32_t kWords = Fused && kFusedLevelLdsWords > kQuadLeafLdsWords ? kFusedLevelLdsWords : kQuadLeafLdsWords;
    __shared__ __attribute__((aligned(16))) uint32_t lds[kWords];
    leaf_quad_wg<Fused>(a, blockIdx.x, lds);
}

// ---- one round of workgroups and a short tail ----------------------------------------
// Just above T0 = 2^16 * K chunks, the lane-per-chunk leaf would put a further workgroup of
// 256 * K chunks on some CUs beside one round of them, and those CUs would take a whole
// workgroup's time longer. Here the chunks past T0 (at most 2^15: two quad workgroups per CU)
// run on quads in the same launch: a quad workgroup hashes 64 chunks with 16 block steps of
// ~273 VALU instructions per wave, against 256 * K chunks and 16 * K steps of ~680 per wave for
// a lane workgroup, so it adds at most 40% (K = 1), 20% (K = 2) or 10% (K = 4) to a CU's issue
// work instead of a whole round (measured, the split adds 8-10 us to the time of the round
// alone: 64 -> 65 MiB 40.3 -> 49.1 us, where the ordinary leaf takes 59.5 us; 128 -> 129 MiB
// 60.3 -> 68.7 us against 83.8; 256 -> 257 MiB 103.4 -> 112.4 us against 122.7). The quad
// workgroups come first in the grid, so that they are dispatched first and spread over the
// CUs; with 130 VGPRs a SIMD holds three waves, so a CU with two quad workgroups takes one
// lane workgroup of the round. T0 is a power
// of two, so the first T0 chunks are the left subtree of the message's tree and the tail the
// right one (page "BLAKE3 on GPU", section "Merkle tree reduction": the left subtree holds the
// largest power of two of chunks below the whole).
template <uint32_t K>
constexpr uint32_t split_lds_words() {
    return kQuadLeafLdsWords > leaf_lds_words<K, false>() ? kQuadLeafLdsWords : leaf_lds_words<K, false>();
}

template <uint32_t K>
__global__ __launch_bounds__(kLeafLanes) void leaf_split_kernel(SplitLeafArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[split_lds_words<K>()];
    if (blockIdx.x < a.tail_wgs) {
        leaf_quad_wg<false>(a.tail, blockIdx.x, lds);
    } else {
        // At four chunks per lane the lane workgroups run four times as long as the quads
        // beside them and set the time, but the quad workgroups, dispatched first, are the
        // older waves and would be issued first; a higher priority for the lane workgroups
        // lets the quads fill the cycles they leave (257 MiB 112.7 -> 110.1 us on MI355X; at
        // one or two chunks per lane the tail is as long as the round and it lost: 65 MiB
        // 48.3 -> 50.2 us, 129 MiB 68.3 -> 69.0 us).
        if (K == 4) __builtin_amdgcn_s_setprio(1);
        leaf_uniform_wg<K, false, false>(a.main, blockIdx.x - a.tail_wgs, lds);
    }
}

// The two subtrees of leaf_split_kernel's message as two segments of one tree of C lanes: the
// 256 main group CVs at positions 0..255, the tail's tail_n <= C / 2 at C / 2 .. (a position
// that is a multiple of the next power of two of tail_n, so that every level pairs nodes of
// one segment only). Neither is final: each segment's CV goes to LDS (`roots`) for the
// parent compression after the tree.
template <uint32_t C>
struct SplitSegs {
    uint32_t tail_n;
    uint32_t key[8];
    uint32_t mode_flag;
    uint32_t *roots;  // LDS, 2 x 8 words

    __device__ uint32_t used_positions() const { return C / 2 + tail_n; }
    __device__ uint32_t root_bit() const { return 0u; }
    __device__ int seg_of(uint32_t pos) const {
        if (pos < kLevelLanes) return 0;
        return pos >= C / 2 && pos - C / 2 < tail_n ? 1 : -1;
    }
    __device__ uint32_t start(int s) const { return s == 0 ? 0u : C / 2; }
    __device__ uint32_t count(int s) const { return s == 0 ? kLevelLanes : tail_n; }
    __device__ bool final(int) const { return false; }
    __device__ uint32_t mode() const { return mode_flag; }
    __device__ void key_words(int, uint32_t (&kw)[8]) const {
#pragma unroll
        for (int w = 0; w < 8; ++w) kw[w] = key[w];
    }
    __device__ void emit(int s, const uint32_t (&cv)[8]) const {
#pragma unroll
        for (int w = 0; w < 8; ++w) roots[8 * s + w] = cv[w];
    }
    __device__ void emit_pair(int s, uint32_t j, uint32_t lo, uint32_t hi) const {
        roots[8 * s + j] = lo;
        roots[8 * s + 4 + j] = hi;
    }
};

template <uint32_t C>
__global__ __launch_bounds__(C) void level_split_root_kernel(SplitRootArgs a) {
    static_assert(C / 2 >= kLevelLanes, "the main segment fits below the tail");
    __shared__ uint32_t buf[2][8][C];
    __shared__ __attribute__((aligned(16))) uint32_t roots[16];
    const uint32_t lane = threadIdx.x;
    SplitSegs<C> sg{};
    sg.tail_n = a.tail_n;
#pragma unroll
    for (int w = 0; w < 8; ++w) sg.key[w] = a.key[w];
    sg.mode_flag = a.mode;
    sg.roots = roots;
    uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (lane < kLevelLanes)
        load_cv(cv, a.main_cv + 8 * lane);
    else if (lane >= C / 2 && lane - C / 2 < a.tail_n)
        load_cv(cv, a.tail_cv + 8 * (lane - C / 2));
    tree_reduce<C>(cv, sg, ceil_log2(a.tail_n > kLevelLanes ? a.tail_n : kLevelLanes), buf);
    __syncthreads();  // both subtree CVs are in `roots`
    if (lane < 4) {   // their parent on one quad: words 0..7 the left CV, 8..15 the right one
        const uint32_t j = lane;
        uint32_t moff[28];
#pragma unroll
        for (int r = 0; r < 7; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t) moff[4 * r + t] = (static_cast<uint32_t>(kQuadWord.at[r][t]) >> (4 * j)) & 15u;
        uint32_t va = pick4(a.key[0], a.key[1], a.key[2], a.key[3], j);
        uint32_t vb = pick4(a.key[4], a.key[5], a.key[6], a.key[7], j);
        uint32_t vc = pick4(kIV[0], kIV[1], kIV[2], kIV[3], j);
        uint32_t vd = j == 3u ? a.mode | kParent | a.root_flag : (j == 2u ? kBlockBytes : 0u);  // counter 0
        compress_quad_lds(va, vb, vc, vd, roots, moff);
        store_digest_pair(a.out, j, va ^ vc, vb ^ vd);
    }
}

// Level segments that one workgroup reduces together (fused_batch_level): n of them, in
// slots of 2^lanes_log2 lanes (from kMinSlotLanes to the whole workgroup), read from LDS.
constexpr uint32_t kMinSlotLanes = 4;
constexpr uint32_t kMaxSlots = kLevelLanes / kMinSlotLanes;
struct LevelSlots {
    const Seg *seg;        // LDS, n entries
    uint32_t n;
    uint32_t lanes_log2;
    const uint32_t *keys;  // global, nullptr for default mode
    uint32_t *cv_out;
    uint8_t *digests;
    const uint32_t *slot_key;  // LDS, kMaxSlots x 8 words: slot s's key at 8 * s (keyed mode)

    __device__ uint32_t used_positions() const { return n << lanes_log2; }
    __device__ uint32_t root_bit() const { return kRoot; }
    __device__ int seg_of(uint32_t pos) const {
        const uint32_t s = pos >> lanes_log2;
        return s < n && pos - (s << lanes_log2) < seg_count(seg[s].info) ? static_cast<int>(s) : -1;
    }
    __device__ uint32_t start(int s) const { return static_cast<uint32_t>(s) << lanes_log2; }
    __device__ uint32_t count(int s) const { return seg_count(seg[s].info); }
    __device__ bool final(int s) const { return seg_final(seg[s].info); }
    __device__ uint32_t mode() const { return keys ? kKeyedHash : 0u; }
    __device__ void key_words(int s, uint32_t (&kw)[8]) const {
        if (keys) {
#pragma unroll
            for (int w = 0; w < 8; ++w) kw[w] = slot_key[8 * s + w];
        } else {
#pragma unroll
            for (int w = 0; w < 8; ++w) kw[w] = kIV[w];
        }
    }
    __device__ void emit(int s, const uint32_t (&cv)[8]) const {
        if (final(s)) store_digest(digests + 32ull * seg[s].msg, cv);
        else store_cv(cv_out + 8ull * seg[s].dst, cv);
    }
    __device__ void emit_pair(int s, uint32_t j, uint32_t lo, uint32_t hi) const {
        if (final(s)) store_digest_pair(digests + 32ull * seg[s].msg, j, lo, hi);
        else store_cv_pair(cv_out + 8ull * seg[s].dst, j, lo, hi);
    }
};

template <>
struct EarlyLevelReads<LevelSlots> : std::true_type {};

// The slot of a position is pos >> lanes_log2 (below kMaxSlots for any position of the
// workgroup), so its key is read without waiting for the segment's info.
__device__ __forceinline__ void seg_key_words(const LevelSlots &sg, const NodeRef &, uint32_t pos,
                                              uint32_t (&kw)[8]) {
    sg.key_words(static_cast<int>(pos >> sg.lanes_log2), kw);
}

// Fused first level pass of a batch (BatchLeafArgs::up), called by the whole workgroup after
// its leaf tree has written the CVs of its segments that are not whole messages, with
// device-coherent stores. Each such CV belongs to one segment of the first level pass; its
// segment here takes that level segment's ticket, and the last of them to arrive sets the
// ticket back to zero and reduces the level segment in this workgroup: it loads the level
// segment's CVs with device-coherent loads (the last node the parent of two CVs when a
// message end was split), runs the level tree, and writes the message's digest when the
// level finishes it, else a CV for the next level pass. A workgroup that holds the ends of
// several messages is often the last arrival for several level segments: they are reduced
// together, as many per round as fit in the workgroup's 256 lanes in slots sized to the
// round's largest segment (a ragged batch's level segments hold a few CVs each). The
// ordering is that of fused_levels. `own` (256 words of LDS, free once the leaf tree is
// done) lists the level segments this workgroup took last; `slots` (kMaxSlots entries)
// holds a round's segments, `slot_key` (8 * kMaxSlots words) their keys, and `round` four
// words: the number of segments taken, then a round's slot count, width and tree depth.
__device__ void fused_batch_level(const BatchLeafArgs &a, const Seg *s_seg, uint32_t nseg, uint32_t *lds,
                                  uint32_t *own, uint32_t *round, Seg *slots, uint32_t *slot_key) {
    static_assert(kMaxSlots == kWaveLanes, "one wave plans a round, one lane per slot");
    const uint32_t lane = threadIdx.x;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's CV stores have completed
    if (lane == 0) round[0] = 0;
    __syncthreads();  // ... in every wave, and the leaf tree is done with the LDS
    if (lane < nseg) {
        const Seg g = s_seg[lane];
        if (!seg_final(g.info)) {
            const uint32_t j = a.up[g.dst];
            const uint32_t info = a.lvl_segs[j].info;
            const uint32_t inputs = seg_count(info) + (seg_pair(info) ? 1u : 0u);
            uint32_t *ticket = a.lvl_ctr + j;
            if (__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == inputs) {
                __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                own[atomicAdd(&round[0], 1u)] = j;
            }
        }
    }
    __syncthreads();
    const uint32_t owned = round[0];
    auto buf = reinterpret_cast<uint32_t(*)[8][kLevelLanes]>(lds);
    for (uint32_t o = 0; o < owned;) {
        __syncthreads();  // the previous round is done with `slots`, `slot_key`, `round` and the LDS
        if (lane < kWaveLanes) {
            // wave 0 plans this round: as many of the next segments as fit in the workgroup in
            // slots of equal power-of-two width, the smallest that holds the largest of them (at
            // least kMinSlotLanes lanes, so at most kMaxSlots segments). Lane i looks at the
            // i-th next segment; running maxima of the widths and tree depths over the lanes
            // then say which of them fit.
            const uint32_t i = o + lane;
            const bool valid = i < owned;
            Seg g{0u, 0u, 0u, 0u};
            uint32_t depth = 0;
            if (valid) {
                g = a.lvl_segs[own[i]];
                depth = ceil_log2(seg_count(g.info));
            }
            uint32_t width = depth > ceil_log2(kMinSlotLanes) ? depth : ceil_log2(kMinSlotLanes);
#pragma unroll
            for (uint32_t d = 1; d < kWaveLanes; d <<= 1) {
                const uint32_t w2 = __shfl_up(width, d), d2 = __shfl_up(depth, d);
                if (lane >= d) {
                    width = w2 > width ? w2 : width;
                    depth = d2 > depth ? d2 : depth;
                }
            }
            // (lane + 1) << width grows with the lane, so the lanes that fit are a prefix
            const bool fits = valid && ((lane + 1) << width) <= kLevelLanes;
            const uint32_t r = static_cast<uint32_t>(__popcll(__ballot(fits)));
            if (lane < r) {
                slots[lane] = g;
                if (a.keys) {
                    uint32_t kw[8];
                    load_cv(kw, a.keys + 8ull * g.msg);
#pragma unroll
                    for (int w = 0; w < 8; ++w) slot_key[8 * lane + w] = kw[w];
                }
            }
            if (lane + 1 == (r > 0 ? r : 1u)) {
                round[1] = r;
                round[2] = width;
                round[3] = depth;
            }
        }
        __syncthreads();
        const uint32_t r = round[1], levels = round[3];
        if (r == 0) break;  // not reached: a level segment holds at most kLevelLanes CVs
        LevelSlots sg{slots, r, round[2], a.keys, a.lvl_cv_out, a.digests, slot_key};
        const uint32_t s = lane >> sg.lanes_log2, x = lane - (s << sg.lanes_log2);
        uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (s < r) {
            const Seg g = slots[s];
            const uint32_t cnt = seg_count(g.info);
            if (x < cnt) {
                const uint32_t *src = a.cv_out + 8ull * (g.first + x);
#pragma unroll
                for (int w = 0; w < 8; ++w) cv[w] = load_word_coherent(src + w);
                if (seg_pair(g.info) && x + 1 == cnt) {  // the two halves of a split message end
                    uint32_t left[8], key[8];
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        left[w] = cv[w];
                        cv[w] = load_word_coherent(src + 8 + w);
                    }
                    sg.key_words(static_cast<int>(s), key);
                    parent_left(cv, left, key, sg.mode(), false);
                }
            }
        }
        tree_reduce<kLevelLanes, LevelSlots, true>(cv, sg, levels, buf);
        o += r;
    }
}

// Fused: the first level pass runs in this launch (fused_batch_level); a separate
// instantiation, so that its registers do not weigh on the default leaf.
// LDS of the batch leaf: that of the leaf, and room beside the tree's level buffers for the
// per-position key table, written once the chunk phase is done with the LDS (and in the
// fused level pass, once the leaf tree is done with it, the slots' keys).
template <uint32_t K, bool Staged>
constexpr uint32_t batch_leaf_lds_words() {
    constexpr uint32_t tree = 2 * 8 * kLanes + kPosKeyWords;
    return leaf_lds_words<K, Staged>() > tree ? leaf_lds_words<K, Staged>() : tree;
}

template <uint32_t K, bool Staged, bool Fused>
__global__ __launch_bounds__(kLeafLanes) void leaf_batch_kernel(BatchLeafArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[batch_leaf_lds_words<K, Staged>()];
    __shared__ Seg s_seg[kLanes];
    __shared__ int s_seg_of[kLanes];
    __shared__ uint32_t s_pos_info[kLanes];
    __shared__ uint32_t s_round[4];
    __shared__ Seg s_slots[Fused ? kMaxSlots : 1];
    stage_segments<kLanes>(a.wg_first_seg, a.segs, s_seg, s_seg_of, s_pos_info);
    const uint32_t lane = threadIdx.x;
    const int s = s_seg_of[lane];
    static_assert(8 * kMaxSlots <= kPosKeyWords, "the fused level pass keeps its slots' keys in the key table");
    uint32_t *pos_key = lds + 2 * 8 * kLanes;
    BatchSegs sg{s_seg, s_seg_of, a.keys, a.cv_out, a.digests, Fused, s_pos_info, pos_key};
    uint32_t key[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint8_t *ptr = a.base;
    uint32_t nl = 0, last_len = kChunkBytes;
    uint64_t c0 = 0;
    bool root = false;
    if (s >= 0) {
        const Seg g = s_seg[s];
        const uint64_t mlen = a.msg_len[g.msg];
        const uint64_t msg_chunks = mlen == 0 ? 1 : (mlen + kChunkBytes - 1) / kChunkBytes;
        const uint64_t seg_left = msg_chunks - g.first;  // chunks from the segment start to the message end
        const uint32_t x = lane - seg_lane(g.info);       // node index within the segment
        const uint64_t lane_left = seg_left - static_cast<uint64_t>(x) * K;
        nl = lane_left < K ? static_cast<uint32_t>(lane_left) : K;
        c0 = g.first + static_cast<uint64_t>(x) * K;
        const uint64_t rem = mlen - (c0 + nl - 1) * kChunkBytes;
        last_len = mlen == 0 ? 0u : (rem < kChunkBytes ? static_cast<uint32_t>(rem) : kChunkBytes);
        ptr = a.base + a.msg_off[g.msg] + c0 * kChunkBytes;
        root = seg_final(g.info) && seg_count(g.info) == 1;
        sg.key_words(s, key);
#pragma unroll
        for (int w = 0; w < 8; ++w) cv[w] = key[w];
    }
    if (__ballot(nl != K || last_len != kChunkBytes) == 0) {
        if (Staged) {
            // every lane holds K full chunks: gather the 8 rows each lane loads for
            const uint32_t lw = lane % kWaveLanes;
            const uint64_t my = reinterpret_cast<uint64_t>(ptr);
            GatherRows rows;
#pragma unroll
            for (uint32_t j = 0; j < 8; ++j)
                rows.src[j] = reinterpret_cast<const uint8_t *>(__shfl(my, static_cast<int>(8 * j + (lw >> 3)))) +
                              16 * stage_piece(lw);
            staged_subtree<K>(cv, rows, lds + (lane / kWaveLanes) * (kStageBytes / 4), c0, key, sg.mode(),
                              root ? kRoot : 0u);
        } else {
            direct_subtree<K, false, K == 1>(cv, ptr, c0, key, sg.mode(), root ? kRoot : 0u, lds + lane);
        }
    } else if (nl > 0) {
        // the ends of a batch's messages: whole workgroups of them, often alone on their
        // SIMDs at the end of the grid, so their loads are issued a block ahead
        lane_subtree<K, true, K == 1>(cv, ptr, nl, last_len, c0, key, sg.mode(), root);
    }
    if (K == 1) __builtin_amdgcn_s_setprio(0);  // the turns end with the chunks
    __syncthreads();  // every wave is done with its stage buffer before the tree reuses it
    if (a.keys && s >= 0) {  // the key table, read by the tree levels behind their first barrier
#pragma unroll
        for (int w = 0; w < 8; ++w) pos_key[w * kPosKeyStride + lane] = key[w];
    }
    tree_reduce<kLanes>(cv, sg, a.wg_levels[blockIdx.x], reinterpret_cast<uint32_t(*)[8][kLanes]>(lds));
    if (Fused)
        fused_batch_level(a, s_seg, a.wg_first_seg[blockIdx.x + 1] - a.wg_first_seg[blockIdx.x], lds,
                          reinterpret_cast<uint32_t *>(s_seg_of), s_round, s_slots, pos_key);
}

__global__ __launch_bounds__(kLevelLanes) void level_batch_kernel(BatchLevelArgs a) {
    static_assert(kLevelLanes == kLanes, "the per-position key table is sized for kLanes positions");
    __shared__ uint32_t buf[2][8][kLevelLanes];
    __shared__ Seg s_seg[kLevelLanes];
    __shared__ int s_seg_of[kLevelLanes];
    __shared__ uint32_t s_pos_info[kLevelLanes];
    __shared__ uint32_t s_pos_key[kPosKeyWords];
    stage_segments<kLevelLanes>(a.wg_first_seg, a.segs, s_seg, s_seg_of, s_pos_info);
    const uint32_t lane = threadIdx.x;
    const int s = s_seg_of[lane];
    uint32_t cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    BatchSegs sg{s_seg, s_seg_of, a.keys, a.cv_out, a.digests, false, s_pos_info, s_pos_key};
    if (s >= 0) {
        const Seg g = s_seg[s];
        const uint32_t x = lane - seg_lane(g.info);
        uint32_t key[8];
        sg.key_words(s, key);
        load_cv(cv, a.cv_in + 8ull * (g.first + x));
        if (a.keys) {  // the key table, read by the tree levels behind their first barrier
#pragma unroll
            for (int w = 0; w < 8; ++w) s_pos_key[w * kPosKeyStride + lane] = key[w];
        }
        if (seg_pair(g.info) && x + 1 == seg_count(g.info)) {
            // the message's end was split in two subtrees in pass 0: this node is their parent
            uint32_t left[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) left[w] = cv[w];
            load_cv(cv, a.cv_in + 8ull * (g.first + x + 1));
            parent_left(cv, left, key, sg.mode(), false);
        }
    }
    tree_reduce<kLevelLanes>(cv, sg, a.wg_levels[blockIdx.x], buf);
}

// ---- extended output ------------------------------------------------------------------

// Root node of a one-chunk message: chain its blocks up to the last (one lane; at most
// 15 compressions) and copy the last block zero-padded.
__global__ __launch_bounds__(64) void xof_chunk_root_kernel(ChunkRootArgs a) {
    if (threadIdx.x != 0) return;
    const uint32_t nb = a.len == 0 ? 1u : (a.len + kBlockBytes - 1) / kBlockBytes;
    uint32_t cv[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) cv[w] = a.key[w];
    for (uint32_t b = 0; b + 1 < nb; ++b) {
        uint32_t m[16];
#pragma unroll
        for (int w = 0; w < 16; ++w) m[w] = load_word_bounded(a.in, b * kBlockBytes + 4 * w, a.len);
        compress(cv, m, 0, 0, kBlockBytes, a.mode | (b == 0 ? kChunkStart : 0u));
    }
    const uint32_t off = (nb - 1) * kBlockBytes;
#pragma unroll
    for (int w = 0; w < 16; ++w) a.m_out[w] = load_word_bounded(a.in, off + 4 * w, a.len);
#pragma unroll
    for (int w = 0; w < 8; ++w) a.cv_out[w] = cv[w];
}

// Rotation of a wave-uniform word on the scalar unit (which has no rotate: a shift pair
// and an or). Written as assembly so that the compiler keeps the chain off the VALU.
template <int K>
__device__ __forceinline__ uint32_t srotr(uint32_t x) {
    uint32_t r, t;
    asm("s_lshr_b32 %0, %2, %3\n\ts_lshl_b32 %1, %2, %4\n\ts_or_b32 %0, %0, %1"
        : "=&s"(r), "=&s"(t)
        : "s"(x), "n"(K), "n"(32 - K)
        : "scc");
    return r;
}

// Quarter-round on wave-uniform words, on the scalar unit.
__device__ __forceinline__ void quarter_uniform(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d, uint32_t x,
                                                uint32_t y) {
    a = a + b + x;
    d = srotr<16>(d ^ a);
    c = c + d;
    b = srotr<12>(b ^ c);
    a = a + b + y;
    d = srotr<8>(d ^ a);
    c = c + d;
    b = srotr<7>(b ^ c);
}

// One 64-byte output block per lane: block t is the root compression run with counter t,
// all sixteen output words. Only the counter differs between lanes, and in round 0 it
// enters column 0 (low word) and column 1 (high word, the same for the whole launch).
// Columns 1..3 and the first sum of column 0 therefore read only wave-uniform words and
// run once per wave on the scalar unit, which takes 37 of the block's 688 VALU
// instructions off the vector unit. The stores keep to the requested byte range. A wave
// whose 64 blocks are whole, in range and 16-byte aligned at the destination passes them
// through LDS so that each of its four 16-byte stores writes 1 KiB contiguously (64 lanes
// x 16 B) instead of 16 B every 64 B; the transposition stays inside the wave, whose LDS
// accesses complete in order.
__global__ __launch_bounds__(kXofLanes) void xof_expand_kernel(XofArgs a) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kXofLanes + threadIdx.x;
    if (i >= a.n_blocks) return;
    const uint64_t t = a.first_block + i;
    const uint32_t t_hi = static_cast<uint32_t>(a.first_block >> 32);
    // the root's inputs are the same for every lane and nothing here writes them: scalar loads
    const uint32_t *__restrict__ src_m = a.m;
    uint32_t cv[8], m[16], v[16];
    if (a.cv) {
        const uint32_t *__restrict__ src_cv = a.cv;
#pragma unroll
        for (int w = 0; w < 8; ++w) cv[w] = src_cv[w];
    } else {
#pragma unroll
        for (int w = 0; w < 8; ++w) cv[w] = a.key[w];
    }
#pragma unroll
    for (int w = 0; w < 16; ++w) m[w] = src_m[w];
    // round 0, columns (the schedule of round 0 is the identity)
    v[1] = cv[1], v[5] = cv[5], v[9] = kIV[1], v[13] = t_hi;
    quarter_uniform(v[1], v[5], v[9], v[13], m[2], m[3]);
    v[2] = cv[2], v[6] = cv[6], v[10] = kIV[2], v[14] = a.block_len;
    quarter_uniform(v[2], v[6], v[10], v[14], m[4], m[5]);
    v[3] = cv[3], v[7] = cv[7], v[11] = kIV[3], v[15] = a.flags;
    quarter_uniform(v[3], v[7], v[11], v[15], m[6], m[7]);
    {
        uint32_t &pa = v[0], &pb = v[4], &pc = v[8], &pd = v[12];
        pa = cv[0] + cv[4] + m[0];  // uniform
        pb = cv[4], pc = kIV[0], pd = static_cast<uint32_t>(t);
        pd = rotr(pd ^ pa, 16);
        pc = pc + pd;
        pb = rotr(pb ^ pc, 12);
        pa = pa + pb + m[1];
        pd = rotr(pd ^ pa, 8);
        pc = pc + pd;
        pb = rotr(pb ^ pc, 7);
    }
    rounds_after_columns(v, m);
    uint32_t o[16];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        o[w] = v[w] ^ v[w + 8];
        o[w + 8] = v[w + 8] ^ cv[w];
    }
    // stream bytes [s0, s0 + 64) of this block, clipped to [out_offset, last], `last` being
    // the request's last byte (out_len >= 1 and the request ends at byte 2^64 at the
    // latest, so computing it does not wrap). Every launched block starts at or before
    // `last`, so last - s0 never wraps, where s0 + 64 or the request's end would for the
    // last block of the 2^64-byte stream.
    const uint64_t s0 = kBlockBytes * t, last = a.out_offset + (a.out_len - 1);
    // the wave path (the condition is the same for all lanes of the wave: a wave with
    // lanes past n_blocks, which returned above, never takes it)
    __shared__ uint4 xo[kXofLanes / 64][256];
    const uint64_t w0 = static_cast<uint64_t>(blockIdx.x) * kXofLanes + (threadIdx.x & ~63u);
    const uint64_t ws0 = kBlockBytes * (a.first_block + w0);
    if (w0 + 64 <= a.n_blocks && ws0 >= a.out_offset && last - ws0 >= 64 * kBlockBytes - 1 &&
        (reinterpret_cast<uintptr_t>(a.out) - a.out_offset) % 16 == 0) {
        const uint32_t wv = threadIdx.x >> 6, ln = threadIdx.x & 63u;
        uint4 *row = xo[wv];
        row[4 * ln + 0] = make_uint4(o[0], o[1], o[2], o[3]);
        row[4 * ln + 1] = make_uint4(o[4], o[5], o[6], o[7]);
        row[4 * ln + 2] = make_uint4(o[8], o[9], o[10], o[11]);
        row[4 * ln + 3] = make_uint4(o[12], o[13], o[14], o[15]);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        uint4 *d = reinterpret_cast<uint4 *>(a.out + (ws0 - a.out_offset));
#pragma unroll
        for (int q = 0; q < 4; ++q) d[64 * q + ln] = row[64 * q + ln];
        return;
    }
    if (s0 >= a.out_offset && last - s0 >= kBlockBytes - 1 &&
        reinterpret_cast<uintptr_t>(a.out + (s0 - a.out_offset)) % 16 == 0) {
        uint4 *d = reinterpret_cast<uint4 *>(a.out + (s0 - a.out_offset));
        d[0] = make_uint4(o[0], o[1], o[2], o[3]);
        d[1] = make_uint4(o[4], o[5], o[6], o[7]);
        d[2] = make_uint4(o[8], o[9], o[10], o[11]);
        d[3] = make_uint4(o[12], o[13], o[14], o[15]);
    } else {
        // stream bytes lo .. hi (inclusive) of this block: 1 to 64 of them
        const uint64_t lo = s0 > a.out_offset ? s0 : a.out_offset;
        const uint64_t hi = last - s0 > kBlockBytes - 1 ? s0 + (kBlockBytes - 1) : last;
        const uint32_t count = static_cast<uint32_t>(hi - lo) + 1;
        for (uint32_t i = 0; i < count; ++i) {
            const uint32_t k = static_cast<uint32_t>(lo - s0) + i;
            a.out[lo - a.out_offset + i] = static_cast<uint8_t>(o[k / 4] >> (8 * (k % 4)));
        }
    }
}

}  // namespace

// dst[i] = src[i] for n 16-byte words: the upload of a batch's task table from pinned host
// memory, as a kernel on the caller's stream, so that the kernels after it wait only for
// the stream's own order (a copy-engine transfer costs a wait across engines).
__global__ __launch_bounds__(256) void copy_words16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                           uint64_t n) {
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<uint64_t>(gridDim.x) * 256)
        dst[i] = src[i];
}

hipError_t launch_copy_words16(const void *src, void *dst, uint64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(copy_words16_kernel, dim3(blocks < 512 ? static_cast<uint32_t>(blocks) : 512u), dim3(256), 0,
                       s, static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_words_kernel(uint32_t *p, uint32_t value, uint64_t n) {
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<uint64_t>(gridDim.x) * 256)
        p[i] = value;
}

hipError_t launch_fill_words(uint32_t *p, uint32_t value, uint64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_words_kernel, dim3(blocks < 1024 ? static_cast<uint32_t>(blocks) : 1024u), dim3(256), 0,
                       s, p, value, n);
    return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t *p, uint64_t n, hipStream_t s) { return launch_fill_words(p, 0, n, s); }

hipError_t launch_xof_expand(const XofArgs &a, uint32_t grid, hipStream_t s) {
    hipLaunchKernelGGL(xof_expand_kernel, dim3(grid), dim3(kXofLanes), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_xof_chunk_root(const ChunkRootArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(xof_chunk_root_kernel, dim3(1), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_uniform_leaf(const UniformLeafArgs &a, uint32_t chunks_per_lane, bool staged, uint32_t grid,
                               hipStream_t s) {
    const dim3 g(grid), b(kLeafLanes);
    if (a.levels != 0) {  // fused level passes: direct loads only
        switch (staged ? 0 : chunks_per_lane) {
            case 1: hipLaunchKernelGGL((leaf_uniform_kernel<1, false, true>), g, b, 0, s, a); break;
            case 2: hipLaunchKernelGGL((leaf_uniform_kernel<2, false, true>), g, b, 0, s, a); break;
            case 4: hipLaunchKernelGGL((leaf_uniform_kernel<4, false, true>), g, b, 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (chunks_per_lane * 2 + (staged ? 1 : 0)) {
        case 2: hipLaunchKernelGGL((leaf_uniform_kernel<1, false, false>), g, b, 0, s, a); break;
        case 3: hipLaunchKernelGGL((leaf_uniform_kernel<1, true, false>), g, b, 0, s, a); break;
        case 4: hipLaunchKernelGGL((leaf_uniform_kernel<2, false, false>), g, b, 0, s, a); break;
        case 5: hipLaunchKernelGGL((leaf_uniform_kernel<2, true, false>), g, b, 0, s, a); break;
        case 8: hipLaunchKernelGGL((leaf_uniform_kernel<4, false, false>), g, b, 0, s, a); break;
        case 9: hipLaunchKernelGGL((leaf_uniform_kernel<4, true, false>), g, b, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quad_leaf(const UniformLeafArgs &a, uint32_t grid, hipStream_t s) {
    if (a.levels != 0)
        hipLaunchKernelGGL(leaf_quad_kernel<true>, dim3(grid), dim3(kLeafLanes), 0, s, a);
    else
        hipLaunchKernelGGL(leaf_quad_kernel<false>, dim3(grid), dim3(kLeafLanes), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_split_leaf(const SplitLeafArgs &a, uint32_t chunks_per_lane, hipStream_t s) {
    const dim3 g(a.tail_wgs + a.main.groups), b(kLeafLanes);
    switch (chunks_per_lane) {
        case 1: hipLaunchKernelGGL(leaf_split_kernel<1>, g, b, 0, s, a); break;
        case 2: hipLaunchKernelGGL(leaf_split_kernel<2>, g, b, 0, s, a); break;
        case 4: hipLaunchKernelGGL(leaf_split_kernel<4>, g, b, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_split_root(const SplitRootArgs &a, hipStream_t s) {
    if (a.tail_n == 0 || a.tail_n > 2 * kLevelLanes) return hipErrorInvalidValue;
    if (a.tail_n <= kLevelLanes)
        hipLaunchKernelGGL(level_split_root_kernel<2 * kLevelLanes>, dim3(1), dim3(2 * kLevelLanes), 0, s, a);
    else
        hipLaunchKernelGGL(level_split_root_kernel<4 * kLevelLanes>, dim3(1), dim3(4 * kLevelLanes), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_uniform_level(const UniformLevelArgs &a, uint32_t grid, hipStream_t s) {
    hipLaunchKernelGGL(level_uniform_kernel, dim3(grid), dim3(kLevelLanes), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_batch_leaf(const BatchLeafArgs &a, uint32_t chunks_per_lane, bool staged, bool fused, uint32_t grid,
                             hipStream_t s) {
    const dim3 g(grid), b(kLeafLanes);
    if (fused) {  // direct loads only
        switch (staged ? 0 : chunks_per_lane) {
            case 1: hipLaunchKernelGGL((leaf_batch_kernel<1, false, true>), g, b, 0, s, a); break;
            case 2: hipLaunchKernelGGL((leaf_batch_kernel<2, false, true>), g, b, 0, s, a); break;
            case 4: hipLaunchKernelGGL((leaf_batch_kernel<4, false, true>), g, b, 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (chunks_per_lane * 2 + (staged ? 1 : 0)) {
        case 2: hipLaunchKernelGGL((leaf_batch_kernel<1, false, false>), g, b, 0, s, a); break;
        case 3: hipLaunchKernelGGL((leaf_batch_kernel<1, true, false>), g, b, 0, s, a); break;
        case 4: hipLaunchKernelGGL((leaf_batch_kernel<2, false, false>), g, b, 0, s, a); break;
        case 5: hipLaunchKernelGGL((leaf_batch_kernel<2, true, false>), g, b, 0, s, a); break;
        case 8: hipLaunchKernelGGL((leaf_batch_kernel<4, false, false>), g, b, 0, s, a); break;
        case 9: hipLaunchKernelGGL((leaf_batch_kernel<4, true, false>), g, b, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_batch_level(const BatchLevelArgs &a, uint32_t grid, hipStream_t s) {
    hipLaunchKernelGGL(level_batch_kernel, dim3(grid), dim3(kLevelLanes), 0, s, a);
    return hipGetLastError();
}

}  // namespace b3g
