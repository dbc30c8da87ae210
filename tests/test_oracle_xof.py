"""The oracle's extended output (XOF), CPU only.

What fixes what:
  * Bytes 0..31 of the output stream are the hash: that ties the root node the XOF
    re-runs (the last block of a one-chunk input, else the parent of the two top
    subtrees) and its ROOT flag to the digest, which the Xet cross-check in
    test_oracle_pins.py pins to an independent BLAKE3.
  * The stream is one sequence: a longer request extends a shorter one.
  * Reading from an offset gives the same bytes as the stream read from its start.
  * Every 64-byte output block, both halves, at any counter t: inverting it (final state
    from the block and the root's input chaining value, then the seven rounds run
    backwards by this module's own inverse of G) must give back the state the root
    compression starts from, counter t included. The root's inputs come from the test's
    data (a one-block input) or from the two top subtrees' chaining values (a parent
    root). A second half built from the wrong words, or a block under the wrong counter,
    fails this. No independent extendable-output implementation or printed vector is
    available here, so the pin is this algebraic one, not a cross-check.
"""
import numpy as np
import pytest

import oracle

LENGTHS = [0, 1, 63, 64, 65, 1023, 1024, 1025, 2048, 3000, 5 * 1024 + 7, 64 * 1024 + 1]


def _data(n, seed=5):
    return np.random.Generator(np.random.PCG64(seed)).bytes(n)


@pytest.mark.parametrize("keyed", [False, True])
@pytest.mark.parametrize("n", LENGTHS)
def test_first_32_bytes_are_the_hash(n, keyed):
    data = _data(n)
    key = _data(32, 9) if keyed else None
    assert oracle.hash_xof(data, key, 32) == oracle.hash(data, key)
    assert oracle.hash_xof(data, key, 100)[:32] == oracle.hash(data, key)


@pytest.mark.parametrize("n", [0, 700, 1024, 5000])
def test_longer_output_extends_shorter(n):
    data = _data(n, 11)
    key = _data(32, 12)
    full = oracle.hash_xof(data, key, 1000)
    assert len(full) == 1000
    for k in (0, 1, 31, 32, 33, 63, 64, 65, 128, 199, 999):
        assert oracle.hash_xof(data, key, k) == full[:k]


def test_output_blocks_differ():
    # each 64-byte block comes from a different counter: no block repeats
    out = oracle.hash_xof(_data(3000, 13), None, 64 * 40)
    blocks = {out[64 * i:64 * i + 64] for i in range(40)}
    assert len(blocks) == 40


@pytest.mark.parametrize("n", [0, 100, 1024, 3000])
def test_reading_from_an_offset_matches_the_stream(n):
    data = _data(n, 14)
    key = _data(32, 15)
    full = oracle.hash_xof(data, key, 1200)
    for off in (0, 1, 31, 32, 63, 64, 65, 100, 640, 1000):
        for k in (0, 1, 63, 64, 65, 129):
            if off + k <= len(full):
                assert oracle.hash_xof(data, key, k, offset=off) == full[off:off + k], (off, k)


def test_offsets_past_the_32_bit_block_counter():
    # blocks 2^32 - 1 and 2^32 differ (the counter's high word enters the state) and a read
    # across that boundary is the concatenation of reads on either side
    data = _data(2500, 16)
    base = 64 * (1 << 32)
    a = oracle.hash_xof(data, None, 64, offset=base - 64)
    b = oracle.hash_xof(data, None, 64, offset=base)
    assert a != b
    assert oracle.hash_xof(data, None, 128, offset=base - 64) == a + b
    assert oracle.hash_xof(data, None, 50, offset=base - 20) == a[44:] + b[:30]
    # block t = 2^32 is not block 0: the high word is not dropped
    assert b != oracle.hash_xof(data, None, 64)


# ---- every output block inverts to the root node's documented input state ---------------
#
# The compression is a permutation of its 16-word state followed by a feed-forward. Given an
# output block and the input chaining value h, the final state is v[i+8] = out[i+8] ^ h[i],
# v[i] = out[i] ^ v[i+8]; running the seven rounds backwards must then give back the state
# the specification starts from: h, the first four IV words, the counter's two words, the
# block length and the flags. The test holds its own inverse of G and of the round (never
# the oracle's forward code); a wrong permutation or rotation here could only fail it. It
# checks both halves of every 64-byte block and the counter t of each one, at any t.

_M32 = 0xFFFFFFFF
# The message permutation applied between rounds (the table the Xet cross-check pins
# through the oracle's digests).
_SIGMA = (2, 6, 3, 10, 7, 0, 4, 13, 1, 11, 12, 5, 9, 14, 15, 8)
_COLUMNS = ((0, 4, 8, 12), (1, 5, 9, 13), (2, 6, 10, 14), (3, 7, 11, 15))
_DIAGONALS = ((0, 5, 10, 15), (1, 6, 11, 12), (2, 7, 8, 13), (3, 4, 9, 14))


def _rotl(x, n):
    return ((x << n) | (x >> (32 - n))) & _M32


def _g_inverse(v, a, b, c, d, mx, my):
    # G adds b and mx into a, then xors d with a and rotates it right by 16, adds d into c,
    # xors b with c and rotates it right by 12, then repeats with my and rotations 8 and 7.
    # Undo those eight steps last first.
    v[b] = _rotl(v[b], 7) ^ v[c]
    v[c] = (v[c] - v[d]) & _M32
    v[d] = _rotl(v[d], 8) ^ v[a]
    v[a] = (v[a] - v[b] - my) & _M32
    v[b] = _rotl(v[b], 12) ^ v[c]
    v[c] = (v[c] - v[d]) & _M32
    v[d] = _rotl(v[d], 16) ^ v[a]
    v[a] = (v[a] - v[b] - mx) & _M32


def _initial_state(out_block, h, m):
    """The 16-word state a compression with chaining value h and message words m started
    from, given its 64-byte output block."""
    o = [int.from_bytes(out_block[4 * i:4 * i + 4], "little") for i in range(16)]
    v = [0] * 16
    for i in range(8):
        v[i + 8] = o[i + 8] ^ h[i]
        v[i] = o[i] ^ v[i + 8]
    schedule = [list(m)]
    for _ in range(6):
        schedule.append([schedule[-1][_SIGMA[i]] for i in range(16)])
    for mr in reversed(schedule):
        for i, (a, b, c, d) in enumerate(_DIAGONALS):
            _g_inverse(v, a, b, c, d, mr[8 + 2 * i], mr[9 + 2 * i])
        for i, (a, b, c, d) in enumerate(_COLUMNS):
            _g_inverse(v, a, b, c, d, mr[2 * i], mr[2 * i + 1])
    return v


def _le_words(b):
    return [int.from_bytes(b[4 * i:4 * i + 4], "little") for i in range(len(b) // 4)]


def _root_inputs(data, key):
    """(h, message words, block length, flags) of the root node, from the data itself for a
    one-block input and from the two top subtrees' chaining values for a parent root."""
    h = _le_words(key) if key is not None else oracle.iv()
    mode = oracle.KEYED_HASH if key is not None else 0
    n = len(data)
    if n <= oracle.BLOCK_LEN:
        block = bytes(data) + bytes(oracle.BLOCK_LEN - n)
        return h, _le_words(block), n, mode | oracle.CHUNK_START | oracle.CHUNK_END | oracle.ROOT
    chunks = -(-n // oracle.CHUNK_LEN)
    assert chunks > 1, "one-chunk inputs longer than a block are not covered here"
    left = oracle.left_subtree_chunks(chunks)
    cut = left * oracle.CHUNK_LEN
    lcv = oracle.subtree_cv(data[:cut], 0, key)
    rcv = oracle.subtree_cv(data[cut:], left, key)
    return h, lcv + rcv, oracle.BLOCK_LEN, mode | oracle.PARENT | oracle.ROOT


@pytest.mark.parametrize("keyed", [False, True])
@pytest.mark.parametrize("n", [0, 1, 63, 64, 1025, 2048, 3000, 5 * 1024 + 7])
def test_output_blocks_invert_to_the_root_state(n, keyed):
    data = _data(n, 17)
    key = _data(32, 18) if keyed else None
    h, m, blen, flags = _root_inputs(data, key)
    iv4 = oracle.iv()[:4]
    counters = [0, 1, 2, 3, 17, 255, (1 << 32) - 1, 1 << 32, (1 << 40) + 5]
    for t in counters:
        block = oracle.hash_xof(data, key, 64, offset=64 * t)
        want = list(h) + iv4 + [t & _M32, t >> 32, blen, flags]
        assert _initial_state(block, h, m) == want, (n, keyed, t)
    # a run of consecutive blocks read in one call: block k carries counter k
    stream = oracle.hash_xof(data, key, 64 * 6)
    for t in range(6):
        want = list(h) + iv4 + [t, 0, blen, flags]
        assert _initial_state(stream[64 * t:64 * t + 64], h, m) == want, (n, keyed, t)


def test_inverse_round_undoes_the_oracles_round():
    # the test's inverse against the oracle's forward round on random states: one round
    # forward then back is the identity (this checks the inverse, not the oracle)
    rng = np.random.Generator(np.random.PCG64(19))
    for _ in range(20):
        v = [int(x) for x in rng.integers(0, 1 << 32, 16, dtype=np.uint64)]
        m = [int(x) for x in rng.integers(0, 1 << 32, 16, dtype=np.uint64)]
        w = oracle.round_fn(v, m)
        for i, (a, b, c, d) in enumerate(_DIAGONALS):
            _g_inverse(w, a, b, c, d, m[8 + 2 * i], m[9 + 2 * i])
        for i, (a, b, c, d) in enumerate(_COLUMNS):
            _g_inverse(w, a, b, c, d, m[2 * i], m[2 * i + 1])
        assert w == v
