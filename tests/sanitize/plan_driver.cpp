// Drives the batch planner over random and edge-case batches, for a build under
// AddressSanitizer and UndefinedBehaviorSanitizer, and checks the plan's layout: every
// workgroup's segments sit inside it, aligned to their power of two and in lane order,
// the first-segment index is monotone, and every output CV slot is written once. Exit
// status 1 on a broken plan; the sanitizers end the run on any memory or UB error.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "b3_plan.h"

namespace {
uint64_t rng_state = 0x2545F4914F6CDD1Dull;
uint64_t next_u64() {  // xorshift64
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

int check(const b3g::BatchPlan &plan, const char *what) {
    for (const b3g::PassPlan &p : plan.passes) {
        const uint32_t w = p.workgroups();
        if (p.wg_first_seg.size() != w + 1 || p.wg_first_seg.back() != p.segs.size()) {
            std::fprintf(stderr, "%s: workgroup index size\n", what);
            return 1;
        }
        std::vector<uint8_t> written(p.out_cvs, 0);
        for (uint32_t g = 0; g < w; ++g) {
            if (p.wg_first_seg[g] >= p.wg_first_seg[g + 1]) {
                std::fprintf(stderr, "%s: empty or unordered workgroup %u\n", what, g);
                return 1;
            }
            uint32_t used = 0, level = 0;
            for (uint32_t s = p.wg_first_seg[g]; s < p.wg_first_seg[g + 1]; ++s) {
                const b3g::Seg &sg = p.segs[s];
                const uint32_t lane = sg.info & 0xFFFu, count = ((sg.info >> 12) & 0xFFFu) + 1;
                const uint32_t r = 1u << b3g::ceil_log2_host(count);
                if (lane < used || lane % r != 0 || lane + count > p.lanes) {
                    std::fprintf(stderr, "%s: segment %u misplaced\n", what, s);
                    return 1;
                }
                used = lane + count;
                level = b3g::ceil_log2_host(count) > level ? b3g::ceil_log2_host(count) : level;
                if (!(sg.info & b3g::kSegFinal)) {
                    if (sg.dst >= p.out_cvs || written[sg.dst]) {
                        std::fprintf(stderr, "%s: output slot %u\n", what, sg.dst);
                        return 1;
                    }
                    written[sg.dst] = 1;
                }
            }
            if (p.wg_levels[g] != level) {
                std::fprintf(stderr, "%s: workgroup %u level\n", what, g);
                return 1;
            }
        }
        for (uint64_t i = 0; i < p.out_cvs; ++i)
            if (!written[i]) {
                std::fprintf(stderr, "%s: output slot %llu never written\n", what, (unsigned long long)i);
                return 1;
            }
    }
    return 0;
}
}  // namespace

int main() {
    b3g::BatchPlan plan;
    static const uint32_t ks[] = {1, 2, 4};
    for (int trial = 0; trial < 300; ++trial) {
        const uint64_t n = 1 + next_u64() % 400;
        std::vector<uint64_t> lens(n);
        for (uint64_t &l : lens) {
            const uint64_t kind = next_u64() % 8;
            l = kind < 4 ? next_u64() % 4097                      // tiny
                : kind < 7 ? next_u64() % (2ull << 20)            // up to 2 MiB
                           : next_u64() % (80ull << 20);          // up to 80 MiB: level passes
        }
        const uint32_t k = ks[trial % 3];
        if (b3g::plan_batch(lens.data(), n, 256, k, 256, &plan) != 0) {
            std::fprintf(stderr, "trial %d: planning failed\n", trial);
            return 1;
        }
        if (check(plan, "random batch")) return 1;
    }
    // edge cases: nothing, one empty message, many tiny ones, a message past the limit
    if (b3g::plan_batch(nullptr, 0, 256, 1, 256, &plan) != 0 || !plan.passes.empty()) return 1;
    std::vector<uint64_t> one{0};
    if (b3g::plan_batch(one.data(), 1, 256, 1, 256, &plan) != 0 || check(plan, "empty message")) return 1;
    std::vector<uint64_t> tiny(20000, 17);
    if (b3g::plan_batch(tiny.data(), tiny.size(), 256, 1, 256, &plan) != 0 || check(plan, "tiny")) return 1;
    std::vector<uint64_t> big{5, b3g::kMaxMessageBytes + 1};
    if (b3g::plan_batch(big.data(), big.size(), 256, 1, 256, &plan) != -5) return 1;
    std::puts("planner driver: every plan well formed");
    return 0;
}
