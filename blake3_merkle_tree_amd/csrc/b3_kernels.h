// b3_kernels.h - host-side view of the gfx950 kernels (argument blocks and launchers).
//
// Two kernel families, following the split of the page "BLAKE3 on GPU: 400x faster
// hashing" (qfminer.top), sections "Our implementation", "Kernel 1" and "Kernels 2 and 3":
//   leaf   - every lane compresses one 1 KiB chunk, then the workgroup reduces its chunk
//            chaining values (CVs) as a fused partial Merkle tree and writes one CV per
//            segment (or the digest, when the segment is a whole message).
//   level  - every lane loads one CV of the previous level; the same in-workgroup tree
//            reduction yields one CV per segment; the last launch sets ROOT.
// A "segment" is an aligned group of consecutive tree nodes of one message that a
// workgroup reduces to a single node. Because every split of the BLAKE3 tree over more
// than 2^k nodes falls on a multiple of 2^k (left subtrees are complete powers of two),
// reducing aligned power-of-two groups level by level reproduces the tree exactly.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "b3_plan.h"

namespace b3g {

// Lanes (= tree nodes) per workgroup. Both kernels use 256 lanes (4 wave64s); a leaf lane
// covers K consecutive chunks (a node of the tree K leaves up).
constexpr uint32_t kLeafLanes = 256;
constexpr uint32_t kLevelLanes = 256;

// Uniform batch: n messages of `len` bytes each, message m at base + m * stride (one
// message is n = 1). Geometry follows from blockIdx, so no task table is needed.
//   Case A (lanes_per_msg != 0): a message's nodes fit one workgroup; each message takes
//     lanes_per_msg = R lanes (a power of two), a workgroup holds 256 / R messages and
//     finishes them (digests).
//   Case B (lanes_per_msg == 0): a message spans `groups` workgroups; workgroup w reduces
//     group (w mod groups) of message (w / groups) to one CV at cv_out + 8*w.
// Fused level passes (case B): after writing its group CV a workgroup takes a ticket on
// its level-1 group (256 group CVs of one message); the last of a group to arrive reduces
// it and takes a ticket one level up, until the message's root. At most kMaxLevels steps:
// groups per message <= 2^32.
constexpr uint32_t kMaxLevels = 4;

struct UniformLeafArgs {
    const uint8_t *base;     // message 0 (16-byte aligned)
    uint64_t stride;         // bytes from one message to the next (multiple of 16)
    uint64_t len;            // bytes per message
    uint64_t n_chunks;       // chunks per message: max(1, ceil(len / 1024))
    uint64_t chunk_base;     // counter of chunk 0 of every message (0 for whole messages)
    uint32_t n_msgs;
    uint32_t lanes_per_msg;  // R in case A, 0 in case B
    uint32_t groups;         // workgroups per message in case B
    uint32_t may_root;       // 1: a workgroup holding a whole message finishes it (writes `digests`)
    uint32_t root_flag;      // flag of a finished message's top compression: ROOT, or 0 (subtree CV)
    const uint32_t *keys;    // 8 key words per message, or nullptr: every message uses `key`
    uint32_t key[8];         // key words (or the IV) when keys == nullptr
    uint32_t mode;           // kKeyedHash or 0
    uint32_t *cv_out;
    uint8_t *digests;        // message m's digest at digests + 32*m
    // fused levels (case B only; levels == 0: the leaf's CVs are the result)
    uint32_t levels;                     // level steps after the leaf
    uint32_t *lvl_cv[kMaxLevels];        // [0] == cv_out; [L]: n_msgs * lvl_g[L] CVs, message-major
    uint32_t *lvl_ctr[kMaxLevels];       // [L]: n_msgs * lvl_g[L + 1] tickets, zero on entry and exit
    uint64_t lvl_g[kMaxLevels + 1];      // nodes per message: [0] = groups, [L + 1] = ceil([L] / 256)
};

// Uniform level pass: every message has g_in CVs, contiguous in cv_in (message m's at
// cv_in + 8 * m * g_in). Case A (g_in <= 256): R = next power of two of g_in lanes per
// message, digests out. Case B: g_out = ceil(g_in / 256) workgroups per message, CVs out.
struct UniformLevelArgs {
    const uint32_t *cv_in;
    uint64_t g_in;
    uint32_t n_msgs;
    uint32_t lanes_per_msg;  // R in case A, 0 in case B
    uint32_t g_out;          // case B
    const uint32_t *keys;
    uint32_t key[8];
    uint32_t mode;
    uint32_t root_flag;      // flag of the finishing pass's top compressions: ROOT, or 0 (subtree CVs)
    uint32_t *cv_out;
    uint8_t *digests;
};

// Batch mode: workgroups read their segments (struct Seg, b3_plan.h) from a task table.
__host__ __device__ inline uint32_t seg_lane(uint32_t info) { return info & 0xFFFu; }
__host__ __device__ inline uint32_t seg_count(uint32_t info) { return ((info >> 12) & 0xFFFu) + 1u; }
__host__ __device__ inline bool seg_final(uint32_t info) { return (info & kSegFinal) != 0; }
__host__ __device__ inline bool seg_pair(uint32_t info) { return (info & kSegPair) != 0; }

struct BatchLeafArgs {
    const uint8_t *base;          // message buffer (16-byte aligned)
    const uint64_t *msg_off;      // per message: byte offset from base
    const uint64_t *msg_len;      // per message: byte length
    const uint32_t *keys;         // per message 8 key words, or nullptr for default mode
    const uint32_t *wg_first_seg; // workgroup w owns segments [wg_first_seg[w], wg_first_seg[w+1])
    const uint8_t *wg_levels;     // workgroup w runs wg_levels[w] tree levels
    const Seg *segs;
    uint32_t *cv_out;             // next level array
    uint8_t *digests;             // out + 32*msg for final segments
    // fused first level pass (leaf_batch_kernel<..., Fused>): the last workgroup to deliver
    // a level segment's CVs reduces it in this launch
    const uint32_t *up;           // level segment that takes each CV of cv_out
    const Seg *lvl_segs;          // the first level pass's segments
    uint32_t *lvl_ctr;            // one ticket per level segment, zero on entry and exit
    uint32_t *lvl_cv_out;         // the first level pass's output CVs (for the passes after it)
};

struct BatchLevelArgs {
    const uint32_t *cv_in;        // current level array
    const uint32_t *keys;
    const uint32_t *wg_first_seg;
    const uint8_t *wg_levels;
    const Seg *segs;
    uint32_t *cv_out;
    uint8_t *digests;
};

// chunks_per_lane (K) is 1, 2 or 4: each leaf workgroup covers 256*K chunks. `staged`
// selects the LDS-staged input path for full waves instead of per-lane loads. With
// a.levels != 0 (fused level passes) only per-lane loads are built: staged is rejected.
hipError_t launch_uniform_leaf(const UniformLeafArgs &a, uint32_t chunks_per_lane, bool staged, uint32_t grid,
                               hipStream_t s);
hipError_t launch_uniform_level(const UniformLevelArgs &a, uint32_t grid, hipStream_t s);

// Small inputs: one quad of lanes per chunk, kQuadLeafChunks chunks per workgroup, one
// chunk per node (lanes_per_msg and groups count chunk slots of that workgroup).
constexpr uint32_t kQuadLeafChunks = 64;
hipError_t launch_quad_leaf(const UniformLeafArgs &a, uint32_t grid, hipStream_t s);

// One message a little longer than a power of two T0 = 2^16 * K chunks (K = 1, 2 or 4): the
// leaf groups of the first T0 chunks (256 workgroups of 256 * K chunks, one round on the 256
// CUs) and the tail past T0 on quads (quad leaf groups of kQuadLeafChunks chunks) in one
// launch, the tail's tail_wgs workgroups first. main and tail describe the two parts as
// case-B uniform leaves (may_root = 0: group CVs to their cv_out).
struct SplitLeafArgs {
    UniformLeafArgs main;
    UniformLeafArgs tail;
    uint32_t tail_wgs;
};
hipError_t launch_split_leaf(const SplitLeafArgs &a, uint32_t chunks_per_lane, hipStream_t s);
// Its levels and root in one workgroup: the 256 main group CVs reduce to the left subtree's
// CV and the tail_n tail group CVs (1 .. 512) to the right one's, side by side; their parent,
// with root_flag (ROOT, or 0 for a subtree CV), is written to out (32 bytes).
struct SplitRootArgs {
    const uint32_t *main_cv;
    const uint32_t *tail_cv;
    uint32_t tail_n;
    uint32_t key[8];
    uint32_t mode;
    uint32_t root_flag;
    uint8_t *out;
};
hipError_t launch_split_root(const SplitRootArgs &a, hipStream_t s);

// n 16-byte words from src (device-visible pinned host memory, or device memory) to dst.
hipError_t launch_copy_words16(const void *src, void *dst, uint64_t n, hipStream_t s);
// Sets n 32-bit words to `value` with a kernel, in stream order (a kernel rather than
// hipMemsetAsync, so that a graph that records it replays it as it ran).
hipError_t launch_fill_words(uint32_t *p, uint32_t value, uint64_t n, hipStream_t s);
// Zeroes n words (the tickets of fused levels): launch_fill_words with 0.
hipError_t launch_zero_words(uint32_t *p, uint64_t n, hipStream_t s);
// Extended output: output block t (64 bytes at out + 64*(t - first_block)) is the root
// compression (cv, m, block_len, flags with ROOT) run with counter t; all 16 output words.
constexpr uint32_t kXofLanes = 256;
struct XofArgs {
    const uint32_t *cv;   // device CV words of the root compression, or nullptr: `key`
    uint32_t key[8];
    const uint32_t *m;    // device: the root compression's 16 message words
    uint32_t block_len;
    uint32_t flags;       // includes ROOT
    uint64_t first_block; // counter of the first block of this launch; a launch never
                          // crosses a multiple of 2^32 blocks (one counter high word)
    uint64_t n_blocks;    // blocks of this launch
    uint8_t *out;         // receives stream bytes [out_offset, out_offset + out_len)
    uint64_t out_offset;
    uint64_t out_len;
};
hipError_t launch_xof_expand(const XofArgs &a, uint32_t grid, hipStream_t s);

// Root compression inputs of a one-chunk message (len <= 1024): the CV after all blocks
// but the last (cv_out, 8 words) and the last block, zero-padded (m_out, 16 words).
struct ChunkRootArgs {
    const uint8_t *in;
    uint32_t len;
    uint32_t key[8];
    uint32_t mode;
    uint32_t *cv_out;
    uint32_t *m_out;
};
hipError_t launch_xof_chunk_root(const ChunkRootArgs &a, hipStream_t s);

// fused: a.up etc. are set and the first level pass runs in this launch (direct loads only).
hipError_t launch_batch_leaf(const BatchLeafArgs &a, uint32_t chunks_per_lane, bool staged, bool fused, uint32_t grid,
                             hipStream_t s);
hipError_t launch_batch_level(const BatchLevelArgs &a, uint32_t grid, hipStream_t s);

}  // namespace b3g
