// b3_plan.h - host planner: how a hash (or a batch of hashes) maps onto kernel launches.
//
// Pure C++ (no HIP): the planner decides, for every launch ("pass"), which aligned
// segments of tree nodes each workgroup reduces. Pass 0 is the leaf pass over chunks,
// pass t > 0 reduces the chaining values written by pass t-1. A message whose segment in
// some pass covers all of its remaining nodes is finished by that pass (its top
// compression carries ROOT and its digest is written).
#pragma once

#include <stdint.h>

#include <vector>

namespace b3g {

// Batch task table entry (mirrored byte for byte in device memory).
struct Seg {
    uint32_t msg;    // message index: key (keys + 8*msg) and digest slot (out + 32*msg)
    uint32_t first;  // pass 0: first chunk index within the message; pass t: first input CV
    uint32_t dst;    // index of the resulting CV in the pass's output array (if not final)
    uint32_t info;   // bits 0..11 lane start, bits 12..23 node count - 1, bit 30 pair, bit 31 final
};
static_assert(sizeof(Seg) == 16, "Seg is a 16-byte table entry");

constexpr uint32_t kSegFinal = 1u << 31;
// The segment's last node is the parent of two input CVs, first + count - 1 and
// first + count (the two halves of a message end split in pass 0).
constexpr uint32_t kSegPair = 1u << 30;
inline constexpr uint32_t seg_info(uint32_t lane, uint32_t count, bool final, bool pair = false) {
    return (lane & 0xFFFu) | (((count - 1) & 0xFFFu) << 12) | (final ? kSegFinal : 0u) | (pair ? kSegPair : 0u);
}

// Largest message accepted (bytes): chunk indices of a message fit in 32 bits.
constexpr uint64_t kMaxMessageBytes = 1ull << 42;
// Longest extended output accepted (bytes).
constexpr uint64_t kMaxXofBytes = 1ull << 42;

struct PassPlan {
    uint32_t lanes = 0;                  // lanes (nodes) per workgroup in this pass
    uint32_t chunks_per_lane = 1;        // pass 0: chunks folded into one node by one lane
    std::vector<Seg> segs;               // sorted by workgroup, then by lane start
    std::vector<uint32_t> wg_first_seg;  // W + 1 entries
    std::vector<uint8_t> wg_levels;      // W entries: ceil(log2(largest segment))
    uint64_t in_cvs = 0;                 // size of the input CV array (passes > 0)
    uint64_t out_cvs = 0;                // size of the output CV array
    std::vector<uint32_t> up;            // passes > 0: the segment of this pass that takes input CV c
    uint32_t workgroups() const { return static_cast<uint32_t>(wg_levels.size()); }
};

struct BatchPlan {
    std::vector<PassPlan> passes;
};

uint64_t chunks_of(uint64_t len);       // max(1, ceil(len / 1024))
uint32_t ceil_log2_host(uint64_t n);     // 0 for n <= 1

// Chunks per leaf lane (1, 2 or 4) for an input of `total_chunks` chunks: 4 from 2 GiB
// of input, 1 for smaller inputs so that they keep enough waves in flight.
// BLAKE3_GPU_CHUNKS_PER_LANE (1, 2 or 4) in the environment overrides the choice (for
// tests and benchmarks).
uint32_t choose_chunks_per_lane(uint64_t total_chunks);
// The same for a single message of `chunks` chunks: 4 from 2^21 chunks, below that the K that
// gives the busiest CU the fewest chunks per lane (workgroups placed in turn on the 256 CUs),
// the largest among equals.
uint32_t choose_single_chunks_per_lane(uint64_t chunks);

// A single message of `chunks` chunks just above a power of two T0 = 2^16 * K (K = 4, 2 or
// 1), by at most 2^15 chunks (two quad workgroups per CU), hashes its first T0 chunks as one
// round of 256 leaf workgroups and the rest on quads in the same launch: returns that K, or 0
// for the ordinary leaf. Measured on MI355X (us, ordinary leaf / split): 65 MiB 59.5 / 49.1,
// 80 MiB 59.4 / 50.1, 96 MiB 59.7 / 59.8, 129 MiB 83.8 / 68.7, 144 MiB 84.7 / 69.5, 160 MiB
// 84.9 / 80.2, 257 MiB 122.7 / 112.4, 272 MiB 123.6 / 114.0, 288 MiB 124.1 / 124.4; 64, 128 and
// 256 MiB unchanged (a second quad workgroup per CU pays only at two chunks per lane).
// BLAKE3_GPU_SPLIT_TAIL=0 in the environment turns it off; a forced K turns it off too.
uint32_t split_tail_chunks_per_lane(uint64_t chunks);

// Input path of full leaf waves: per-lane loads (default) or staged through LDS with
// coalesced direct-to-LDS loads when BLAKE3_GPU_STAGING=lds is set in the environment.
bool use_lds_staging();

// Inputs (single messages and uniform batches) of at most this many chunks in total take
// the quad leaf (four lanes per chunk): below it the lane-per-chunk leaf is bound by the
// latency of one lane's 16 sequential compressions, not by the chip's VALU rate. Measured on
// MI355X (us, lane-per-chunk / quad leaf): 20 MiB 40.0 / 38.7, 32 MiB 40.1 / 38.8, 40 MiB
// 41.8 / 52.0; 512 messages of 64 KiB 28.3 / 24.1, 2048 of 16 KiB 26.8 / 22.0.
// BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS in the environment overrides it (0 turns it off).
constexpr uint64_t kQuadLeafMaxChunksDefault = 32768;
uint64_t quad_leaf_max_chunks();

// Fused level passes: the leaf launch reduces the levels itself (last-arrival tickets)
// instead of separate level launches. Single messages and uniform batches: only with
// BLAKE3_GPU_FUSED_LEVELS=1 (measured slower). Batches planned into a task table: the first
// level pass, by default where that pass finishes every message with segments of at most 64
// CVs (measured faster there); BLAKE3_GPU_FUSED_LEVELS=1 or 0 forces it on or off.
bool fuse_uniform_levels();
bool fuse_batch_first_level(const BatchPlan &plan);

// Test hooks for the scratch of a call (stream-ordered device memory). A request of more
// than BLAKE3_GPU_SCRATCH_LIMIT bytes fails with B3G_ENOMEM before any HIP call, as an
// allocation failure would; BLAKE3_GPU_SCRATCH_FILL=<byte> (0..255) fills new scratch
// with that byte before the call's kernels run, so that tests can show that no result
// depends on what the memory held before. Unset, neither changes anything.
uint64_t scratch_limit();   // UINT64_MAX when unset
int scratch_fill_byte();    // -1 when unset

// Batches of equal lengths at evenly spaced offsets skip the planner (their geometry is
// implied); BLAKE3_GPU_BATCH_TABLE=1 in the environment routes them through the task
// table like any other batch (for tests).
bool uniform_batch_disabled();

// The BLAKE3_GPU_* variables above are read from the environment once, when the library
// is loaded; reload_options() reads them again (tests and tools change them between calls).
void reload_options();

// Builds the passes for messages of the given byte lengths. Pass 0 groups
// leaf_lanes * chunks_per_lane chunks per workgroup (one node per lane); later passes
// group level_lanes CVs. Returns 0 (B3G_OK) or a negative b3g_status (B3G_ETOOBIG when a
// message or the task table exceeds the limits).
int plan_batch(const uint64_t *lengths, uint64_t n, uint32_t leaf_lanes, uint32_t chunks_per_lane,
               uint32_t level_lanes, BatchPlan *out);

}  // namespace b3g
