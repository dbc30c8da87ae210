// b3_device.h - BLAKE3 compression on one gfx950 lane.
//
// The compression function of the page "BLAKE3 on GPU: 400x faster hashing" (qfminer.top),
// section "Compression function": a 16-word state built from a 32-byte chaining value,
// four IV words, the 64-bit counter, the block length and the flags, run through seven
// rounds of add/xor/rotate quarter-rounds with the message words permuted from round to
// round, then folded to an 8-word chaining value. Like the page's kernel, one lane runs a
// whole compression in registers (compress); where too few nodes are left to fill the
// lanes, four lanes share one (compress_quad). The constants are the BLAKE3
// specification's.
//
// gfx950 mapping: pure 32-bit integer VALU work. a+b+m is one v_add3_u32, each rotation
// one v_alignbit_b32 (or v_perm_b32 for the byte-multiple amounts), each xor one
// v_xor_b32: 12 VALU instructions per quarter-round, 680 per compression including the
// final fold. Nothing here is a contraction, so the matrix cores are not used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace b3g {

constexpr uint32_t kChunkBytes = 1024;
constexpr uint32_t kBlockBytes = 64;
constexpr uint32_t kBlocksPerChunk = kChunkBytes / kBlockBytes;

// Domain-separation flag bits (BLAKE3 specification's flag table).
constexpr uint32_t kChunkStart = 1u << 0;
constexpr uint32_t kChunkEnd = 1u << 1;
constexpr uint32_t kParent = 1u << 2;
constexpr uint32_t kRoot = 1u << 3;
constexpr uint32_t kKeyedHash = 1u << 4;

// Initial value: the first 32 bits of the fractional parts of the square roots of the
// first eight primes.
constexpr uint32_t kIV[8] = {0x6A09E667u, 0xBB67AE85u, 0x3C6EF372u, 0xA54FF53Au,
                             0x510E527Fu, 0x9B05688Cu, 0x1F83D9ABu, 0x5BE0CD19u};

// Message schedule. Between rounds BLAKE3 permutes the 16 message words (new word i is
// old word kPerm[i]). Instead of moving registers, round r reads message word
// kSchedule.at[r][i] at slot i, where at[0] is the identity and at[r+1][i] =
// at[r][kPerm[i]]; after unrolling every index is a compile-time constant, so the
// permutation costs no instructions.
struct Schedule {
    uint8_t at[7][16];
};
constexpr Schedule make_schedule() {
    constexpr uint8_t kPerm[16] = {2, 6, 3, 10, 7, 0, 4, 13, 1, 11, 12, 5, 9, 14, 15, 8};
    Schedule s{};
    for (int i = 0; i < 16; ++i) s.at[0][i] = static_cast<uint8_t>(i);
    for (int r = 1; r < 7; ++r)
        for (int i = 0; i < 16; ++i) s.at[r][i] = s.at[r - 1][kPerm[i]];
    return s;
}
constexpr Schedule kSchedule = make_schedule();

__device__ __forceinline__ uint32_t rotr(uint32_t x, uint32_t k) {
    return __builtin_amdgcn_alignbit(x, x, k);
}

// Quarter-round on (a, b, c, d) with message words x, y.
__device__ __forceinline__ void quarter(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d, uint32_t x,
                                        uint32_t y) {
    a = a + b + x;
    d = rotr(d ^ a, 16);
    c = c + d;
    b = rotr(b ^ c, 12);
    a = a + b + y;
    d = rotr(d ^ a, 8);
    c = c + d;
    b = rotr(b ^ c, 7);
}

// Message word read at slot I of round R (a compile-time index, see kSchedule).
template <int R, int I>
__device__ __forceinline__ uint32_t mw(const uint32_t (&m)[16]) {
    constexpr int k = kSchedule.at[R][I];
    return m[k];
}

// ---- four quarter-rounds in lockstep ----------------------------------------------------
// The four quarter-rounds of a column step (S = 0) or a diagonal step (S = 1) are
// independent. They run in lockstep: each of a quarter-round's twelve instructions is issued
// for all four before the next, with a scheduling barrier after every such group, so that
// every instruction reads a value written four instructions earlier. Left to itself the
// compiler chains one quarter-round's instructions back to back, and a dependent VALU
// instruction waits for its operand: a wave with no other wave on its SIMD to fill those
// cycles then issues at about 80% of the rate (MI355X clock probe of the leaf: a 64-lane
// block step took 1.53 us with one wave per SIMD against 1.35 us with four).
__device__ __forceinline__ void lockstep_fence() { __builtin_amdgcn_sched_barrier(0); }

template <class F>
__device__ __forceinline__ void for_quarters(F &&f) {
    f(std::integral_constant<int, 0>{});
    f(std::integral_constant<int, 1>{});
    f(std::integral_constant<int, 2>{});
    f(std::integral_constant<int, 3>{});
    lockstep_fence();
}

// Quarter-round I of step S works on a = v[I], b = v[4 + (I + S) % 4], c = v[8 + (I + 2S) % 4],
// d = v[12 + (I + 3S) % 4] with the message words at slots 8S + 2I and 8S + 2I + 1.
template <int S, int I>
struct Quarter {
    static constexpr int a = I, b = 4 + (I + S) % 4, c = 8 + (I + 2 * S) % 4, d = 12 + (I + 3 * S) % 4;
    static constexpr int x = 8 * S + 2 * I, y = x + 1;
};

// a += b + x, d = (d ^ a) >>> r1, c += d, b = (b ^ c) >>> r2: the first (x, 16, 12) or the
// second (y, 8, 7) half of the quarter-rounds of step S, in lockstep.
template <int R, int S, bool Second>
__device__ __forceinline__ void half_quarters(uint32_t (&v)[16], const uint32_t (&m)[16]) {
    constexpr uint32_t r1 = Second ? 8 : 16, r2 = Second ? 7 : 12;
    for_quarters([&](auto i) {
        using Q = Quarter<S, decltype(i)::value>;
        v[Q::a] = v[Q::a] + v[Q::b] + mw<R, Second ? Q::y : Q::x>(m);
    });
    for_quarters([&](auto i) {
        using Q = Quarter<S, decltype(i)::value>;
        v[Q::d] ^= v[Q::a];
    });
    for_quarters([&](auto i) {
        using Q = Quarter<S, decltype(i)::value>;
        v[Q::d] = rotr(v[Q::d], r1);
    });
    for_quarters([&](auto i) {
        using Q = Quarter<S, decltype(i)::value>;
        v[Q::c] += v[Q::d];
    });
    for_quarters([&](auto i) {
        using Q = Quarter<S, decltype(i)::value>;
        v[Q::b] ^= v[Q::c];
    });
    for_quarters([&](auto i) {
        using Q = Quarter<S, decltype(i)::value>;
        v[Q::b] = rotr(v[Q::b], r2);
    });
}

template <int R, int S>
__device__ __forceinline__ void quarters(uint32_t (&v)[16], const uint32_t (&m)[16]) {
    half_quarters<R, S, false>(v, m);
    half_quarters<R, S, true>(v, m);
}

template <int R>
__device__ __forceinline__ void round_r(uint32_t (&v)[16], const uint32_t (&m)[16]) {
    quarters<R, 0>(v, m);  // columns
    quarters<R, 1>(v, m);  // diagonals
}

// cv <- first half of compress(cv, m, counter, block_len, flags).
__device__ __forceinline__ void compress(uint32_t (&cv)[8], const uint32_t (&m)[16], uint32_t counter_lo,
                                         uint32_t counter_hi, uint32_t block_len, uint32_t flags) {
    uint32_t v[16] = {cv[0],  cv[1],  cv[2],  cv[3],      cv[4],      cv[5],     cv[6],     cv[7],
                      kIV[0], kIV[1], kIV[2], kIV[3], counter_lo, counter_hi, block_len, flags};
    round_r<0>(v, m);
    round_r<1>(v, m);
    round_r<2>(v, m);
    round_r<3>(v, m);
    round_r<4>(v, m);
    round_r<5>(v, m);
    round_r<6>(v, m);
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = v[i] ^ v[i + 8];
}

// ---- chained blocks: the chaining value kept unfolded ---------------------------------
// Within a chunk, block i+1 starts from block i's output cv[j] = s[j] ^ s[j+8] (s: the 16
// state words after the last round). That fold need not be computed: in the first round
// only the column quarter-rounds read cv, and there a = cv[j], b = cv[4+j] appear in
// a + b + x and b ^ c. With gfx950's three-input ops, (s[j] ^ s[j+8]) + ((s[4+j] ^
// s[12+j]) + x) is two v_xad_u32 and s[4+j] ^ s[12+j] ^ c one v_bitop3_b32, against two
// xors, one v_add3_u32 and one xor: 4 instructions fewer per chained compression (676;
// the first block of a chunk starts from the state (cv, 0) and takes 684).

// (a ^ b) + c in one instruction. Both three-input forms are written as assembly: the
// compiler would otherwise share a ^ b between the sum and the xor below and bring back the
// separate fold.
__device__ __forceinline__ uint32_t xad(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_xad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// a ^ b ^ c in one instruction (v_bitop3_b32 with truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// The rest of round 0 and rounds 1..6 on v, whose columns have already been mixed.
__device__ __forceinline__ void rounds_after_columns(uint32_t (&v)[16], const uint32_t (&m)[16]) {
    quarters<0, 1>(v, m);
    round_r<1>(v, m);
    round_r<2>(v, m);
    round_r<3>(v, m);
    round_r<4>(v, m);
    round_r<5>(v, m);
    round_r<6>(v, m);
}

// v <- the state after compressing block m from the chaining value fold(s). The columns of
// round 0 read cv[j] = s[j] ^ s[j+8] and cv[4+j] = s[4+j] ^ s[12+j] without folding them,
// in lockstep like the other steps: a = cv[j] + (cv[4+j] + x) is two v_xad_u32, the first
// b ^ c one v_bitop3_b32.
__device__ __forceinline__ void compress_chained(const uint32_t (&s)[16], const uint32_t (&m)[16],
                                                 uint32_t counter_lo, uint32_t counter_hi, uint32_t block_len,
                                                 uint32_t flags, uint32_t (&v)[16]) {
    v[8] = kIV[0], v[9] = kIV[1], v[10] = kIV[2], v[11] = kIV[3];
    v[12] = counter_lo, v[13] = counter_hi, v[14] = block_len, v[15] = flags;
    uint32_t t[4];
    for_quarters([&](auto i) {
        constexpr int j = decltype(i)::value;
        t[j] = xad(s[4 + j], s[12 + j], mw<0, 2 * j>(m));
    });
    for_quarters([&](auto i) {
        constexpr int j = decltype(i)::value;
        v[j] = xad(s[j], s[8 + j], t[j]);
    });
    for_quarters([&](auto i) {
        constexpr int j = decltype(i)::value;
        v[12 + j] ^= v[j];
    });
    for_quarters([&](auto i) {
        constexpr int j = decltype(i)::value;
        v[12 + j] = rotr(v[12 + j], 16);
    });
    for_quarters([&](auto i) {
        constexpr int j = decltype(i)::value;
        v[8 + j] += v[12 + j];
    });
    for_quarters([&](auto i) {
        constexpr int j = decltype(i)::value;
        v[4 + j] = xor3(s[4 + j], s[12 + j], v[8 + j]);
    });
    for_quarters([&](auto i) {
        constexpr int j = decltype(i)::value;
        v[4 + j] = rotr(v[4 + j], 12);
    });
    half_quarters<0, 0, true>(v, m);
    rounds_after_columns(v, m);
}

// The chaining value of a state: cv[i] = s[i] ^ s[i+8].
__device__ __forceinline__ void fold_state(uint32_t (&cv)[8], const uint32_t (&s)[16]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = s[i] ^ s[i + 8];
}

// All sixteen output words of the compression (extended output): words 0..7 as in
// compress, words 8..15 = v[i+8] ^ cv[i].
__device__ __forceinline__ void compress_xof(const uint32_t (&cv)[8], const uint32_t (&m)[16], uint32_t counter_lo,
                                             uint32_t counter_hi, uint32_t block_len, uint32_t flags,
                                             uint32_t (&out)[16]) {
    uint32_t v[16] = {cv[0],  cv[1],  cv[2],  cv[3],      cv[4],      cv[5],     cv[6],     cv[7],
                      kIV[0], kIV[1], kIV[2], kIV[3], counter_lo, counter_hi, block_len, flags};
    round_r<0>(v, m);
    round_r<1>(v, m);
    round_r<2>(v, m);
    round_r<3>(v, m);
    round_r<4>(v, m);
    round_r<5>(v, m);
    round_r<6>(v, m);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        out[i] = v[i] ^ v[i + 8];
        out[i + 8] = v[i + 8] ^ cv[i];
    }
}

// ---- one compression on four lanes ---------------------------------------------------
// Lane j (0..3) of a quad (four consecutive lanes, all active) holds column j of the
// state: a = v[j], b = v[4+j], c = v[8+j], d = v[12+j]. In a round each lane runs the
// quarter-round of its column, then the quarter-round of the diagonal through its own b:
// diagonal j - 1 (mod 4), which takes a from lane j - 1, c from lane j + 1 and d from lane
// j + 2 (DPP quad_perm moves); after it the three rows move back. That is 7 x (24 + 6) VALU
// instructions per lane instead of 680 on one lane, for work whose node count leaves lanes
// idle anyway.
//
// Why b stays: each quarter-round is one dependent chain, and the next one starts with
// a + b. Row b is written by the chain's last instruction, so a move of b would sit on the
// chain (and a DPP read of a register written just before needs wait states); rows a, d
// and c are final two to five instructions earlier, so their moves are issued while the
// chain goes on. The moves are kept as plain DPP moves (quad_move) rather than folded into
// the instructions that use them, which would put the DPP read back on the chain with its
// wait states. A single-wave microbenchmark on MI355X: 1008 cycles per quad compression
// against 1208 with rows b, c and d moving.
//
// Lane j reads 4 message words per round: slots 2j, 2j+1 (column) and 8+2i, 9+2i with
// i = (j + 3) mod 4 (its diagonal) of the round's schedule. kQuadWord.at[r][t] packs, 4
// bits per lane, the message word index that lane j reads as its t-th word of round r.
struct QuadWords {
    uint16_t at[7][4];
};
constexpr QuadWords make_quad_words() {
    QuadWords q{};
    for (int r = 0; r < 7; ++r)
        for (int t = 0; t < 4; ++t) {
            uint32_t packed = 0;
            for (int j = 0; j < 4; ++j) {
                const int diag = (j + 3) & 3;
                const int slot = (t < 2 ? 2 * j + t : 8 + 2 * diag + (t - 2));
                packed |= static_cast<uint32_t>(kSchedule.at[r][slot]) << (4 * j);
            }
            q.at[r][t] = static_cast<uint16_t>(packed);
        }
    return q;
}
constexpr QuadWords kQuadWord = make_quad_words();

// Lane j of the quad takes x from lane (j + k) mod 4 (DPP quad_perm, k = 1, 2, 3). The
// source lane is always in the quad, so no lane keeps an old value: with bound_ctrl and
// no old operand the move needs no initialised destination.
template <int K>
__device__ __forceinline__ uint32_t quad_take(uint32_t x) {
    constexpr int ctrl = ((0 + K) & 3) | (((1 + K) & 3) << 2) | (((2 + K) & 3) << 4) | (((3 + K) & 3) << 6);
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), ctrl, 0xF, 0xF, true));
}

// quad_take as a separate move instruction: the empty asm hands its user a register the
// compiler cannot trace back to the move, so the move is not combined into that user.
template <int K>
__device__ __forceinline__ uint32_t quad_move(uint32_t x) {
    uint32_t y = quad_take<K>(x);
    asm volatile("" : "+v"(y));
    return y;
}

// Quarter-round on (a, b, c, d) with message words x, y, after which lane j holds a from
// lane j + KA, c from lane j + KC and d from lane j + KD (mod 4); each move is issued as
// soon as its row has its final value.
template <int KA, int KC, int KD>
__device__ __forceinline__ void quarter_then_move(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d, uint32_t x,
                                                  uint32_t y) {
    a = a + b + x;
    d = rotr(d ^ a, 16);
    c = c + d;
    b = rotr(b ^ c, 12);
    a = a + b + y;
    d ^= a;
    const uint32_t an = quad_move<KA>(a);
    d = rotr(d, 8);
    c += d;
    const uint32_t dn = quad_move<KD>(d);
    b ^= c;
    const uint32_t cn = quad_move<KC>(c);
    b = rotr(b, 7);
    a = an;
    c = cn;
    d = dn;
}

// One round on a quad with this lane's four message words of the round: the column
// quarter-round, then the diagonal one (a from lane j - 1, c from j + 1, d from j + 2),
// then the rows back to their columns.
__device__ __forceinline__ void quad_round_words(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d, uint32_t x0,
                                                 uint32_t x1, uint32_t x2, uint32_t x3) {
    quarter_then_move<3, 1, 2>(a, b, c, d, x0, x1);
    quarter_then_move<1, 3, 2>(a, b, c, d, x2, x3);
}

template <int R>
__device__ __forceinline__ void quad_round(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d,
                                           const uint32_t (&m)[28]) {
    quad_round_words(a, b, c, d, m[4 * R + 0], m[4 * R + 1], m[4 * R + 2], m[4 * R + 3]);
}

// The seven rounds on a quad; m[4r + t] is this lane's t-th message word of round r
// (word index kQuadWord.at[r][t] >> 4j & 15). Afterwards this lane's output words are
// j (a ^ c) and 4 + j (b ^ d).
__device__ __forceinline__ void compress_quad(uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d,
                                              const uint32_t (&m)[28]) {
    quad_round<0>(a, b, c, d, m);
    quad_round<1>(a, b, c, d, m);
    quad_round<2>(a, b, c, d, m);
    quad_round<3>(a, b, c, d, m);
    quad_round<4>(a, b, c, d, m);
    quad_round<5>(a, b, c, d, m);
    quad_round<6>(a, b, c, d, m);
}

// x[j] for a lane-varying j in 0..3, by selects (no indexed register access).
__device__ __forceinline__ uint32_t pick4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t j) {
    const uint32_t lo = (j & 1u) ? x1 : x0, hi = (j & 1u) ? x3 : x2;
    return (j & 2u) ? hi : lo;
}

}  // namespace b3g
