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
// Packing. A full group fills a workgroup alone. Smaller groups are bucketed by the next
// power of two R of their size (largest first, in one linear pass) and laid out back to
// back; because the sizes are non-increasing powers of two, every group then starts at a
// multiple of its own R, which keeps the in-workgroup pairing from mixing groups.
#include "b3_plan.h"

#include <stdlib.h>

#include <algorithm>

namespace b3g {

namespace {
constexpr int kOk = 0;
constexpr int kTooBig = -5;

uint32_t next_pow2(uint32_t n) {
    uint32_t r = 1;
    while (r < n) r <<= 1;
    return r;
}

struct Group {
    uint32_t msg, first, count, dst;
    bool final;
};

// Lays groups out over workgroups of `lanes` lanes (a power of two).
int pack(const std::vector<Group> &groups, uint32_t lanes, PassPlan *p) {
    p->lanes = lanes;  // g.count is in nodes (lanes)
    // bucket the partial groups by log2 of their power of two (stable within a bucket)
    const uint32_t top = ceil_log2_host(lanes);
    std::vector<uint64_t> bucket_size(top + 2, 0);
    uint64_t full = 0;
    for (const Group &g : groups) {
        if (g.count == lanes) ++full;
        else ++bucket_size[ceil_log2_host(g.count)];
    }
    std::vector<uint64_t> bucket_at(top + 2, 0);  // largest power first
    uint64_t pos = 0;
    for (int b = static_cast<int>(top); b >= 0; --b) {
        bucket_at[b] = pos;
        pos += bucket_size[b];
    }
    std::vector<uint32_t> order(pos);
    p->segs.reserve(groups.size());
    p->wg_first_seg.reserve(full + pos / 2 + 2);
    p->wg_levels.reserve(full + pos / 2 + 1);
    for (size_t i = 0; i < groups.size(); ++i) {
        const Group &g = groups[i];
        if (g.count == lanes) {
            p->wg_first_seg.push_back(static_cast<uint32_t>(p->segs.size()));
            p->wg_levels.push_back(static_cast<uint8_t>(ceil_log2_host(g.count)));
            p->segs.push_back(Seg{g.msg, g.first, g.dst, seg_info(0, g.count, g.final)});
        } else {
            order[bucket_at[ceil_log2_host(g.count)]++] = static_cast<uint32_t>(i);
        }
    }
    uint32_t offset = lanes;  // forces a new workgroup for the first partial group
    for (uint32_t i : order) {
        const Group &g = groups[i];
        const uint32_t r = next_pow2(g.count);
        if (offset + r > lanes) {
            p->wg_first_seg.push_back(static_cast<uint32_t>(p->segs.size()));
            p->wg_levels.push_back(0);
            offset = 0;
        }
        p->segs.push_back(Seg{g.msg, g.first, g.dst, seg_info(offset, g.count, g.final)});
        uint8_t &lv = p->wg_levels.back();
        lv = std::max<uint8_t>(lv, static_cast<uint8_t>(ceil_log2_host(g.count)));
        offset += r;
    }
    if (p->segs.size() >= (1ull << 32) || p->wg_levels.size() >= (1ull << 31)) return kTooBig;
    p->wg_first_seg.push_back(static_cast<uint32_t>(p->segs.size()));
    return kOk;
}
}  // namespace

uint64_t chunks_of(uint64_t len) { return len == 0 ? 1 : (len + 1023) / 1024; }

uint32_t choose_chunks_per_lane(uint64_t total_chunks) {
    if (const char *e = getenv("BLAKE3_GPU_CHUNKS_PER_LANE")) {
        const int k = atoi(e);
        if (k == 1 || k == 2 || k == 4) return static_cast<uint32_t>(k);
    }
    // Four chunks per lane from 2 GiB of input: it cuts the lane-sparse top of each
    // workgroup tree and the fold work by 4x once the 1024-chunk workgroups are many rounds
    // of the chip. Measured on MI355X (ms at K = 1 / 2 / 4): 512 MiB 0.197 / 0.197 / 0.206,
    // 1 GiB 0.362 / 0.360 / 0.368, 2 GiB 0.699 / 0.704 / 0.696, 4 GiB 1.416 / 1.390 / 1.384,
    // 8 GiB 2.988 / 2.808 / 2.768; below 2 GiB the extra workgroups of K = 1 win.
    if (total_chunks >= (1ull << 21)) return 4;
    return 1;
}

uint64_t quad_leaf_max_chunks() {
    if (const char *e = getenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS")) return strtoull(e, nullptr, 10);
    return kQuadLeafMaxChunksDefault;
}

bool fused_levels_enabled() {
    // Off by default: measured on MI355X, the ticket zeroing launch and each workgroup's
    // wait for its coherent stores and ticket cost more than the level launches they
    // replace (4 GiB: 1.369 vs 1.351 ms; 1 MiB: 37.0 vs 31.6 us; 256 MiB: 122 vs 113 us).
    const char *e = getenv("BLAKE3_GPU_FUSED_LEVELS");
    return e != nullptr && e[0] == '1' && e[1] == 0;
}

bool uniform_batch_disabled() {
    const char *e = getenv("BLAKE3_GPU_BATCH_TABLE");
    return e != nullptr && e[0] == '1' && e[1] == 0;
}

bool use_lds_staging() {
    const char *e = getenv("BLAKE3_GPU_STAGING");
    return e != nullptr && e[0] == 'l' && e[1] == 'd' && e[2] == 's' && e[3] == 0;
}

uint32_t ceil_log2_host(uint64_t n) {
    return n <= 1 ? 0u : 64u - static_cast<uint32_t>(__builtin_clzll(n - 1));
}

int plan_batch(const uint64_t *lengths, uint64_t n, uint32_t leaf_lanes, uint32_t chunks_per_lane,
               uint32_t level_lanes, BatchPlan *out) {
    out->passes.clear();
    if (n == 0) return kOk;
    if (n >= (1ull << 32)) return kTooBig;
    // nodes[i]: node count of message i entering the current pass (0 once finished)
    std::vector<uint64_t> nodes(n);
    for (uint64_t i = 0; i < n; ++i) {
        if (lengths[i] > kMaxMessageBytes) return kTooBig;
        nodes[i] = chunks_of(lengths[i]);
    }
    // in_base[i]: where message i's input CVs start in the current pass's input array
    std::vector<uint64_t> in_base(n, 0), out_base(n, 0);
    for (uint32_t pass = 0;; ++pass) {
        // a pass-0 node is a lane's run of chunks_per_lane chunks; later nodes are CVs
        const uint64_t per_node = pass == 0 ? chunks_per_lane : 1;
        const uint64_t lanes = pass == 0 ? leaf_lanes : level_lanes;
        const uint64_t span = lanes * per_node;  // units (chunks or CVs) per full group
        // all three are powers of two: shifts instead of divisions in the per-message loop
        const uint32_t node_shift = ceil_log2_host(per_node), span_shift = ceil_log2_host(span);
        std::vector<Group> groups;
        groups.reserve(pass == 0 ? n : n / 4 + 16);
        uint64_t out_cvs = 0;
        for (uint64_t i = 0; i < n; ++i) {
            if (nodes[i] == 0) continue;
            const uint64_t ngroups = (nodes[i] + span - 1) >> span_shift;
            const bool final = ngroups == 1;
            out_base[i] = out_cvs;
            if (!final) out_cvs += ngroups;
            for (uint64_t k = 0; k < ngroups; ++k) {
                const uint64_t first = (pass == 0 ? 0 : in_base[i]) + k * span;
                const uint64_t units = std::min<uint64_t>(span, nodes[i] - k * span);
                const uint64_t count = (units + per_node - 1) >> node_shift;
                if (first >= (1ull << 32) || out_base[i] + k >= (1ull << 32)) return kTooBig;
                groups.push_back(Group{static_cast<uint32_t>(i), static_cast<uint32_t>(first),
                                       static_cast<uint32_t>(count),
                                       final ? 0u : static_cast<uint32_t>(out_base[i] + k), final});
            }
            nodes[i] = final ? 0 : ngroups;
        }
        if (groups.empty()) break;
        PassPlan p;
        p.chunks_per_lane = static_cast<uint32_t>(per_node);
        p.in_cvs = pass == 0 ? 0 : out->passes.back().out_cvs;
        p.out_cvs = out_cvs;
        const int rc = pack(groups, static_cast<uint32_t>(lanes), &p);
        if (rc != kOk) return rc;
        out->passes.push_back(std::move(p));
        in_base.swap(out_base);
    }
    return kOk;
}

}  // namespace b3g
