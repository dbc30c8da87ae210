// b3_plan.cpp - batch planner (see b3_plan.h).
//
// Grouping. Pass 0 cuts message i (n_i chunks) into groups of L0 consecutive chunks
// starting at chunk 0; pass t cuts the m_i CVs left by pass t-1 into groups of L
// consecutive CVs. Every group is a complete power-of-two subtree except possibly the
// last, and because the BLAKE3 tree splits any node over more than 2^k leaves at a
// multiple of 2^k (page "BLAKE3 on GPU: 400x faster hashing", section "BLAKE3": the left
// subtree is complete and at least as large as the right), the tree over the group
// roots is the BLAKE3 tree of the message, one level up.
//
// Split message ends. In pass 0 a message's last group, when it is not the message's
// only group, holds more nodes than half a workgroup and is not a complete power of two,
// would fill a workgroup alone with idle lanes. It is cut instead into its left subtree
// (the largest power of two below its node count: the BLAKE3 tree's left child of that
// group's root) and the rest, two groups with two output CVs; in pass 1 the message's
// last node is their parent, which the lane holding that node computes before the
// workgroup's tree (the segment's pair bit). This keeps the lanes of pass 0 dense
// without changing the tree or the number of passes.
//
// Packing. Every group takes R lanes, the next power of two of its node count (a full
// group: the whole workgroup). Groups are bucketed by R and laid out back to back, the
// largest R first and in message order within a bucket; because the sizes are
// non-increasing powers of two that divide the workgroup, every group starts at a
// multiple of its own R (which keeps the in-workgroup pairing from mixing groups) and
// never straddles two workgroups. A group's lane position is therefore a prefix sum: one
// pass over the messages counts the groups per bucket, a second writes each task entry
// in place, and the workgroup boundaries follow from the bucket layout.
#include "b3_plan.h"

#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <memory>


namespace b3g {

namespace {
constexpr int kOk = 0;
constexpr int kTooBig = -5;
constexpr uint32_t kMaxBuckets = 13;  // lanes per workgroup <= 4096

uint32_t floor_log2_host(uint64_t n) { return 63u - static_cast<uint32_t>(__builtin_clzll(n)); }

// Calls f(first, count, bucket, dst_offset, final, pair) for the groups of one message in
// one pass (see the grouping and split rules above). `nodes`: the message's units
// entering the pass; `first0`: its first unit's index in the pass input; `pair_end`: its
// last node is a pair; `split`: set when its end is split. dst_offset is the group's
// output CV relative to the message's first one.
template <class F>
inline void for_each_group(uint64_t nodes, uint64_t first0, uint32_t per_node_shift, uint32_t span_shift,
                           uint64_t lanes, bool may_split, bool pair_end, bool *split, F &&f) {
    const uint64_t span = 1ull << span_shift;
    const uint64_t ngroups = (nodes + span - 1) >> span_shift;
    const bool final = ngroups == 1;
    for (uint64_t k = 0; k + 1 < ngroups; ++k)
        f(first0 + k * span, lanes, floor_log2_host(lanes), k, false, false);
    const uint64_t k = ngroups - 1;
    const uint64_t tail_units = nodes - k * span;
    const uint64_t count = (tail_units + (1ull << per_node_shift) - 1) >> per_node_shift;
    *split = may_split && !final && 2 * count > lanes && (count & (count - 1)) != 0;
    if (*split) {
        const uint32_t lb = floor_log2_host(count);
        const uint64_t left = 1ull << lb;
        f(first0 + k * span, left, lb, k, false, false);
        f(first0 + k * span + (left << per_node_shift), count - left, ceil_log2_host(count - left), k + 1, false,
          false);
    } else {
        f(first0 + k * span, count, ceil_log2_host(count), k, final, pair_end);
    }
}
}  // namespace

// The BLAKE3_GPU_* test hooks, read from the environment once when the library is loaded
// (and again on reload_options), so that no call reads the environment.
namespace {
struct Options {
    std::atomic<uint32_t> chunks_per_lane{0};  // 0: chosen by input size
    std::atomic<uint64_t> quad_leaf_max_chunks{kQuadLeafMaxChunksDefault};
    std::atomic<uint64_t> scratch_limit{UINT64_MAX};
    std::atomic<int> scratch_fill{-1};
    std::atomic<int> fused_levels{-1};  // -1 the default choice, 0 never, 1 wherever the form exists
    std::atomic<bool> batch_table{false};
    std::atomic<bool> lds_staging{false};
    std::atomic<bool> split_tail{true};
};
Options g_options;

bool env_is(const char *name, const char *value) {
    const char *e = getenv(name);
    return e != nullptr && strcmp(e, value) == 0;
}

void read_options() {
    Options &o = g_options;
    uint32_t k = 0;
    if (const char *e = getenv("BLAKE3_GPU_CHUNKS_PER_LANE")) {
        const int v = atoi(e);
        if (v == 1 || v == 2 || v == 4) k = static_cast<uint32_t>(v);
    }
    o.chunks_per_lane.store(k, std::memory_order_relaxed);
    const char *q = getenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS");
    o.quad_leaf_max_chunks.store(q ? strtoull(q, nullptr, 10) : kQuadLeafMaxChunksDefault, std::memory_order_relaxed);
    const char *lim = getenv("BLAKE3_GPU_SCRATCH_LIMIT");
    o.scratch_limit.store(lim == nullptr || lim[0] < '0' || lim[0] > '9' ? UINT64_MAX : strtoull(lim, nullptr, 10),
                          std::memory_order_relaxed);
    int fill = -1;
    if (const char *f = getenv("BLAKE3_GPU_SCRATCH_FILL")) {
        if (f[0] != 0) {
            char *end = nullptr;
            const long v = strtol(f, &end, 0);
            if (*end == 0 && v >= 0 && v <= 255) fill = static_cast<int>(v);
        }
    }
    o.scratch_fill.store(fill, std::memory_order_relaxed);
    o.fused_levels.store(env_is("BLAKE3_GPU_FUSED_LEVELS", "1") ? 1 : env_is("BLAKE3_GPU_FUSED_LEVELS", "0") ? 0 : -1,
                         std::memory_order_relaxed);
    o.batch_table.store(env_is("BLAKE3_GPU_BATCH_TABLE", "1"), std::memory_order_relaxed);
    o.lds_staging.store(env_is("BLAKE3_GPU_STAGING", "lds"), std::memory_order_relaxed);
    o.split_tail.store(!env_is("BLAKE3_GPU_SPLIT_TAIL", "0"), std::memory_order_relaxed);
}

struct ReadAtLoad {
    ReadAtLoad() { read_options(); }
} g_read_at_load;
}  // namespace

void reload_options() { read_options(); }

uint64_t chunks_of(uint64_t len) { return len == 0 ? 1 : (len + 1023) / 1024; }

uint32_t choose_chunks_per_lane(uint64_t total_chunks) {
    if (const uint32_t k = g_options.chunks_per_lane.load(std::memory_order_relaxed)) return k;
    // Four chunks per lane from 2 GiB of input: it cuts the lane-sparse top of each
    // workgroup tree and the fold work by 4x once the 1024-chunk workgroups are many rounds
    // of the chip. Measured on MI355X (ms at K = 1 / 2 / 4): 512 MiB 0.197 / 0.197 / 0.206,
    // 1 GiB 0.362 / 0.360 / 0.368, 2 GiB 0.699 / 0.704 / 0.696, 4 GiB 1.416 / 1.390 / 1.384,
    // 8 GiB 2.988 / 2.808 / 2.768; below 2 GiB the extra workgroups of K = 1 win.
    if (total_chunks >= (1ull << 21)) return 4;
    return 1;
}

uint32_t choose_single_chunks_per_lane(uint64_t chunks) {
    if (const uint32_t k = g_options.chunks_per_lane.load(std::memory_order_relaxed)) return k;
    // A single message's leaf takes about as long as its busiest CU: with the workgroups
    // placed in turn on the 256 CUs, the CU that holds the most of them, each worth K chunks
    // per lane (the last, partial one only as many as its lanes hold: min(K, its chunks)).
    // K is the one that minimises that, the largest among equals (fewer workgroups, trees and
    // level CVs). Measured on MI355X (us at K = 1 / 2 / 4), the choice in brackets: 64 MiB
    // 43.4 / 60.0 / 101.8 [1], 128 MiB 67.8 / 64.1 / - [2], 192 MiB 89.1 / 105.2 / 104.0 [1],
    // 256 MiB 109.0 / 106.6 / 104.3 [4], 320 MiB 131.1 / 147.2 / 185.1 [1], 384 MiB 153.5 /
    // 150.6 / 186.9 [2], 448 MiB 173.1 / 187.0 / 188.0 [1], 512 MiB 193.2 / 188.4 / 190.1 [4],
    // 640 MiB 236.5 / 229.3 / 266.1 [2], 1 GiB 357.2 / 349.9 / 350.4 [4], 2 GiB 690.2 / 673.7 /
    // 671.8 [4]. From 2^21 chunks (2 GiB) K is 4, as for batches: the rounds are many there,
    // the level CVs fewest, and the fixed scratch of the entry point that allocates nothing
    // is sized for it. Batches do not use this rule: with K > 1 most of their waves hold
    // message ends (1000 messages of 100,000 bytes 55.1 / 65.4 us at K = 1 / 2, 256 ragged
    // messages of 122 MiB in all 76.7 / 116.0).
    if (chunks >= (1ull << 21)) return 4;
    constexpr uint64_t kCUs = 256, kWgLanes = 256;
    uint64_t best_work = UINT64_MAX;
    uint32_t best = 1;
    for (uint32_t k = 1; k <= 4; k *= 2) {
        const uint64_t span = kWgLanes * k;
        const uint64_t wgs = (chunks + span - 1) / span;
        const uint64_t last = chunks - (wgs - 1) * span;  // chunks of the last workgroup
        const uint64_t q = (wgs - 1) / kCUs, rem = (wgs - 1) % kCUs;  // the last one's round and CU
        const uint64_t work = rem > 0 ? (q + 1) * k : q * k + (last < k ? last : k);
        if (work <= best_work) {
            best_work = work;
            best = k;
        }
    }
    return best;
}

uint32_t split_tail_chunks_per_lane(uint64_t chunks) {
    if (!g_options.split_tail.load(std::memory_order_relaxed)) return 0;
    if (g_options.chunks_per_lane.load(std::memory_order_relaxed) != 0) return 0;  // a test forces K
    for (uint32_t k = 4; k >= 1; k /= 2) {
        const uint64_t t0 = (1ull << 16) * k;
        if (chunks > t0 && chunks - t0 <= (1ull << 15)) return k;
    }
    return 0;
}

uint64_t quad_leaf_max_chunks() { return g_options.quad_leaf_max_chunks.load(std::memory_order_relaxed); }
uint64_t scratch_limit() { return g_options.scratch_limit.load(std::memory_order_relaxed); }
int scratch_fill_byte() { return g_options.scratch_fill.load(std::memory_order_relaxed); }
int fused_levels_setting() { return g_options.fused_levels.load(std::memory_order_relaxed); }

bool fuse_uniform_levels() { return fused_levels_setting() == 1; }

bool fuse_batch_first_level(const BatchPlan &plan) {
    if (plan.passes.size() < 2) return false;
    const int setting = fused_levels_setting();
    if (setting >= 0) return setting == 1;
    // Measured on MI355X: fused where the first level pass finishes every message and its
    // segments are small (the workgroups holding message ends, last to finish, each reduce
    // a few short level segments together: 256 ragged messages of 0 B-1 MiB 80.7 -> 77.8 us);
    // a level segment of more CVs makes the grid's end wait for its tree (a 300 MiB message
    // in a batch: 150.3 -> 154.3 us).
    // Only over one round of leaf workgroups: over many, every workgroup's wait for its
    // stores and ticket costs more than the launch saves (1024 messages of ~1 MiB: 390.1 ->
    // 391.3 us).
    if (plan.passes.size() != 2 || plan.passes[0].workgroups() > 1024) return false;
    for (const Seg &g : plan.passes[1].segs)
        if (((g.info >> 12) & 0xFFFu) + 1u + ((g.info & kSegPair) ? 1u : 0u) > 64) return false;
    return true;
}
bool uniform_batch_disabled() { return g_options.batch_table.load(std::memory_order_relaxed); }
bool use_lds_staging() { return g_options.lds_staging.load(std::memory_order_relaxed); }

uint32_t ceil_log2_host(uint64_t n) {
    return n <= 1 ? 0u : 64u - static_cast<uint32_t>(__builtin_clzll(n - 1));
}

int plan_batch(const uint64_t *lengths, uint64_t n, uint32_t leaf_lanes, uint32_t chunks_per_lane,
               uint32_t level_lanes, BatchPlan *out) {
    out->passes.clear();
    if (n == 0) return kOk;
    if (n >= (1ull << 32)) return kTooBig;
    // The messages still open entering a pass, in message order; each pass keeps, in place,
    // those that go on to the next.
    struct Open {
        uint64_t nodes;     // units entering the pass (chunks in pass 0, CVs after)
        uint64_t in_base;   // where its input CVs start in the pass's input array
        uint64_t out_base;  // where its output CVs start in the pass's output array
        uint32_t msg;
        bool pair_end;      // its last node in this pass is the parent of its last two input CVs
        bool split;         // its end is split in this pass
    };
    std::unique_ptr<Open[]> open(new Open[n]);
    uint64_t n_open = n;
    for (uint64_t i = 0; i < n; ++i) {
        if (lengths[i] > kMaxMessageBytes) return kTooBig;
        open[i] = Open{chunks_of(lengths[i]), 0, 0, static_cast<uint32_t>(i), false, false};
    }
    for (uint32_t pass = 0; n_open > 0; ++pass) {
        // a pass-0 node is a lane's run of chunks_per_lane chunks; later nodes are CVs
        const uint64_t per_node = pass == 0 ? chunks_per_lane : 1;
        const uint64_t lanes = pass == 0 ? leaf_lanes : level_lanes;
        const uint32_t top = floor_log2_host(lanes);
        if (top >= kMaxBuckets) return kTooBig;
        const uint32_t node_shift = ceil_log2_host(per_node), span_shift = top + node_shift;
        const bool may_split = pass == 0;
        // groups per bucket (bucket b: groups of 2^b lanes) and each message's output CVs
        uint64_t bucket_n[kMaxBuckets] = {};
        uint64_t out_cvs = 0;
        for (uint64_t j = 0; j < n_open; ++j) {
            Open &m = open[j];
            bool sp = false, final = false;
            for_each_group(m.nodes, m.in_base, node_shift, span_shift, lanes, may_split, m.pair_end, &sp,
                           [&](uint64_t, uint64_t, uint32_t b, uint64_t, bool fin, bool) {
                               ++bucket_n[b];
                               final = fin;
                           });
            m.split = sp;
            m.out_base = out_cvs;
            if (!final) out_cvs += ((m.nodes + (1ull << span_shift) - 1) >> span_shift) + (sp ? 1 : 0);
        }
        uint64_t total = 0;
        for (uint32_t b = 0; b <= top; ++b) total += bucket_n[b];
        if (total >= (1ull << 32) || out_cvs >= (1ull << 32)) return kTooBig;
        // bucket layout, largest groups first: first task entry and first lane position
        uint64_t seg_at[kMaxBuckets], lane_at[kMaxBuckets], seg_pos = 0, lane_pos = 0;
        for (int b = static_cast<int>(top); b >= 0; --b) {
            seg_at[b] = seg_pos;
            lane_at[b] = lane_pos;
            seg_pos += bucket_n[b];
            lane_pos += bucket_n[b] << b;
        }
        const uint64_t workgroups = (lane_pos + lanes - 1) >> top;
        // one launch per pass, and a launch holds at most 2^32 - 1 work-items
        if (workgroups > 0xFFFFFFFFull / lanes) return kTooBig;
        PassPlan p;
        p.lanes = static_cast<uint32_t>(lanes);
        p.chunks_per_lane = static_cast<uint32_t>(per_node);
        p.in_cvs = pass == 0 ? 0 : out->passes.back().out_cvs;
        p.out_cvs = out_cvs;
        // workgroup boundaries: a workgroup starts at every multiple of `lanes`, with the
        // group that begins there (the largest of the workgroup: its tree's level count)
        p.wg_first_seg.reserve(workgroups + 1);
        p.wg_levels.reserve(workgroups);
        for (int b = static_cast<int>(top); b >= 0; --b) {
            const uint64_t l0 = lane_at[b], l1 = l0 + (bucket_n[b] << b);
            for (uint64_t at = (l0 + lanes - 1) & ~(lanes - 1); at < l1; at += lanes) {
                p.wg_first_seg.push_back(static_cast<uint32_t>(seg_at[b] + ((at - l0) >> b)));
                p.wg_levels.push_back(static_cast<uint8_t>(b));
            }
        }
        p.wg_first_seg.push_back(static_cast<uint32_t>(total));
        // task entries in place; the messages that go on move to the front of `open`
        p.segs.resize(total);
        Seg *segs = p.segs.data();
        bool too_big = false;  // a unit index past 32 bits
        uint64_t kept = 0;
        for (uint64_t j = 0; j < n_open; ++j) {
            const Open m = open[j];
            bool sp = false;
            for_each_group(m.nodes, m.in_base, node_shift, span_shift, lanes, may_split, m.pair_end, &sp,
                           [&](uint64_t first, uint64_t count, uint32_t b, uint64_t k, bool fin, bool pair) {
                               const uint64_t lane = lane_at[b];
                               lane_at[b] += 1ull << b;
                               too_big |= first >= (1ull << 32);
                               segs[seg_at[b]++] =
                                   Seg{m.msg, static_cast<uint32_t>(first),
                                       fin ? 0u : static_cast<uint32_t>(m.out_base + k),
                                       seg_info(static_cast<uint32_t>(lane & (lanes - 1)),
                                                static_cast<uint32_t>(count), fin, pair)};
                           });
            // next pass: a message's nodes are its groups (a split end counts once)
            const uint64_t ngroups = (m.nodes + (1ull << span_shift) - 1) >> span_shift;
            if (ngroups > 1) open[kept++] = Open{ngroups, m.out_base, 0, m.msg, m.split, false};
        }
        if (too_big) return kTooBig;
        n_open = kept;
        if (pass > 0) {  // which segment takes each input CV (a pair node's segment takes two)
            p.up.assign(p.in_cvs, 0);
            for (uint64_t j = 0; j < total; ++j) {
                const uint32_t info = segs[j].info;
                const uint64_t first = segs[j].first, n_in = ((info >> 12) & 0xFFFu) + 1u + ((info & kSegPair) ? 1u : 0u);
                for (uint64_t c = first; c < first + n_in && c < p.in_cvs; ++c) p.up[c] = static_cast<uint32_t>(j);
            }
        }
        out->passes.push_back(std::move(p));
    }
    return kOk;
}

}  // namespace b3g
