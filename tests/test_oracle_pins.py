"""Pins of the CPU oracle to facts outside itself (CPU only, no GPU).

What fixes what:
  * IV ............ closed form (fractional parts of square roots of the first 8 primes).
  * G, rotation amounts, IV, column/diagonal layout of a round ..... a BLAKE2s built on the
    oracle's round function must equal Python's hashlib.blake2s (BLAKE2s shares all four;
    its own message schedule and parameter block are RFC 7693's).
  * The whole keyed hash (message permutation, flag values, counter / length / flag state
    words, chunk chaining, tree) ..... equality with the Xet protocol's hasher (hf_xet) on
    single-Xet-chunk files of 1 B to 127 KiB. When hf_xet is not importable those parts
    are parity unpinned by this module (only the internal consistency checks remain).
  * Tree shape ..... the two rules and the 13 = 8+4+1 worked example of the page
    "BLAKE3 on GPU: 400x faster hashing" (sections "BLAKE3" and "Merkle tree reduction").
  * Chunk and parent parameters ..... the page's description: 16 sequential 64-byte block
    compressions per 1 KiB chunk, CHUNK_START first, CHUNK_END last, per-chunk counter
    ("Compression function"); parents with counter 0, block length 64 and
    KEYED_HASH | PARENT ("Merkle tree reduction"); ROOT on the final compression only
    ("Kernels 2 and 3").
"""
import hashlib
import math
import os
import struct
import tempfile

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MASK = 0xFFFFFFFF


def _rng_bytes(seed, n):
    return np.random.Generator(np.random.PCG64(seed)).bytes(n)


def _key_words(key):
    return list(struct.unpack("<8I", key))


# ---------------------------------------------------------------- IV closed form

def test_iv_is_sqrt_primes():
    primes = [2, 3, 5, 7, 11, 13, 17, 19]
    # floor(frac(sqrt(p)) * 2^32) == isqrt(p * 2^64) mod 2^32, exactly in integers.
    expected = [math.isqrt(p << 64) & MASK for p in primes]
    assert oracle.iv() == expected


# ---------------------------------------------------------------- BLAKE2s on the oracle's round

# BLAKE2s message schedule sigma, RFC 7693 section 2.7 (ten rows).
_SIGMA = [
    [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15],
    [14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3],
    [11, 8, 12, 0, 5, 2, 15, 13, 10, 14, 3, 6, 7, 1, 9, 4],
    [7, 9, 3, 1, 13, 12, 11, 14, 2, 6, 5, 10, 4, 0, 15, 8],
    [9, 0, 5, 7, 2, 4, 10, 15, 14, 1, 11, 12, 6, 8, 3, 13],
    [2, 12, 6, 10, 0, 11, 8, 3, 4, 13, 7, 5, 15, 14, 1, 9],
    [12, 5, 1, 15, 14, 13, 4, 10, 0, 7, 6, 3, 9, 2, 8, 11],
    [13, 11, 7, 14, 12, 1, 3, 9, 5, 0, 15, 4, 8, 6, 2, 10],
    [6, 15, 14, 9, 11, 3, 0, 8, 12, 2, 13, 7, 1, 4, 10, 5],
    [10, 2, 8, 4, 7, 6, 1, 5, 15, 11, 9, 14, 3, 12, 13, 0],
]


def _blake2s_on_oracle(data: bytes, key: bytes = b"", outlen: int = 32) -> bytes:
    """BLAKE2s (RFC 7693) whose G / round / IV are the oracle's."""
    iv = oracle.iv()
    h = list(iv)
    h[0] ^= 0x01010000 ^ (len(key) << 8) ^ outlen
    blocks = []
    if key:
        blocks.append(key + b"\0" * (64 - len(key)))
    for i in range(0, len(data), 64):
        blocks.append(data[i:i + 64])
    if not blocks:
        blocks = [b""]
    counter = 0
    for bi, blk in enumerate(blocks):
        last = bi == len(blocks) - 1
        if key and bi == 0:
            counter += 64
        else:
            counter += len(blk)
        m = list(struct.unpack("<16I", blk + b"\0" * (64 - len(blk))))
        v = h + iv
        v[12] ^= counter & MASK
        v[13] ^= (counter >> 32) & MASK
        if last:
            v[14] ^= MASK
        for r in range(10):
            v = oracle.round_fn(v, [m[_SIGMA[r][i]] for i in range(16)])
        h = [h[i] ^ v[i] ^ v[i + 8] for i in range(8)]
    return struct.pack("<8I", *h)[:outlen]


@pytest.mark.parametrize("n", [0, 1, 3, 55, 63, 64, 65, 127, 128, 129, 1000])
def test_blake2s_built_on_oracle_round_matches_hashlib(n):
    data = _rng_bytes(100 + n, n)
    assert _blake2s_on_oracle(data) == hashlib.blake2s(data).digest()
    key = _rng_bytes(200 + n, 32)
    assert _blake2s_on_oracle(data, key) == hashlib.blake2s(data, key=key).digest()


# ---------------------------------------------------------------- independent BLAKE3 (Xet)

# The Xet protocol's published 32-byte key for hashing data chunks.
_XET_DATA_KEY = bytes([102, 151, 245, 119, 91, 149, 80, 222, 49, 53, 203, 172, 165, 151, 24, 28,
                       157, 228, 33, 16, 155, 235, 43, 88, 180, 208, 176, 75, 147, 173, 242, 41])


def _xet_cases():
    cases = []
    with open(os.path.join(GOLDEN, "xet_single_chunk_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                n, seed = line.split()
                cases.append((int(n), int(seed)))
    return cases


def _xet_hex(digest: bytes) -> str:
    return "".join(digest[8 * i:8 * i + 8][::-1].hex() for i in range(4))


def test_oracle_matches_independent_blake3_via_xet():
    hf_xet = pytest.importorskip("hf_xet")
    cases = _xet_cases()
    assert len(cases) >= 10
    with tempfile.TemporaryDirectory() as d:
        paths, datas = [], []
        for n, seed in cases:
            data = _rng_bytes(seed, n)
            p = os.path.join(d, f"in_{n}_{seed}.bin")
            with open(p, "wb") as f:
                f.write(data)
            paths.append(p)
            datas.append(data)
        infos = hf_xet.hash_files(paths)
    for (n, seed), data, info in zip(cases, datas, infos):
        chunk_hash = oracle.hash(data, _XET_DATA_KEY)
        file_hash = oracle.hash(chunk_hash, bytes(32))
        assert info.hash == _xet_hex(file_hash), f"length {n} seed {seed}"
        # the recursive form is checked against the same independent values
        assert oracle.hash_recursive(data, _XET_DATA_KEY) == chunk_hash


# ---------------------------------------------------------------- tree shape rules

def test_left_subtree_obeys_both_rules_and_is_unique():
    for n in range(2, 5000):
        k = oracle.left_subtree_chunks(n)
        assert k & (k - 1) == 0, "left subtree must be complete: a power-of-two chunk count"
        assert k < n
        assert k >= n - k, "left subtree must hold at least as many chunks as the right"
        allowed = [1 << e for e in range(64) if (1 << e) < n and (1 << e) >= n - (1 << e)]
        assert allowed == [k], "the two rules admit exactly one split"


def _chunk_cvs(data, key_words, mode, n):
    return [oracle.chunk_cv(key_words, mode, data[1024 * j:1024 * (j + 1)], j, is_root=False)
            for j in range(n)]


def _perfect(cvs, kw, mode):
    while len(cvs) > 1:
        cvs = [oracle.parent_cv(kw, mode, cvs[i], cvs[i + 1]) for i in range(0, len(cvs), 2)]
    return cvs[0]


def test_page_example_13_leaves():
    with open(os.path.join(GOLDEN, "tree_13_chunks.txt")) as f:
        spec = {ln.split(":", 1)[0].strip(): ln.split(":", 1)[1].strip()
                for ln in f if ln.strip() and not ln.startswith("#")}
    assert spec["leaves"] == "13"
    assert spec["root"] == "P(T8[0..8), P(T4[8..12), C12))"
    key = _rng_bytes(13, 32)
    kw = _key_words(key)
    mode = oracle.KEYED_HASH
    data = _rng_bytes(14, 13 * 1024 - 100)  # last chunk partial
    c = _chunk_cvs(data, kw, mode, 13)
    t8 = _perfect(c[0:8], kw, mode)
    t4 = _perfect(c[8:12], kw, mode)
    root = oracle.parent_cv(kw, mode, t8, oracle.parent_cv(kw, mode, t4, c[12]), is_root=True)
    assert oracle.hash(data, key) == struct.pack("<8I", *root)
    # left-to-right chaining would be a different (wrong) tree: the test is sensitive to it
    wrong = oracle.parent_cv(kw, mode, oracle.parent_cv(kw, mode, t8, t4), c[12], is_root=True)
    assert struct.pack("<8I", *wrong) != oracle.hash(data, key)


# ---------------------------------------------------------------- chunk / parent parameters

def test_chunk_is_sixteen_chained_block_compressions():
    key = _rng_bytes(21, 32)
    kw = _key_words(key)
    data = _rng_bytes(22, 1024)
    cv = kw
    for b in range(16):
        m = list(struct.unpack("<16I", data[64 * b:64 * b + 64]))
        flags = oracle.KEYED_HASH
        if b == 0:
            flags |= oracle.CHUNK_START
        if b == 15:
            flags |= oracle.CHUNK_END | oracle.ROOT
        cv = oracle.compress(cv, m, 0, 64, flags)[:8]
    assert oracle.hash(data, key) == struct.pack("<8I", *cv)


def test_parent_parameters_counter0_len64_keyed_parent():
    key = _rng_bytes(31, 32)
    kw = _key_words(key)
    data = _rng_bytes(32, 2048)
    c0 = oracle.chunk_cv(kw, oracle.KEYED_HASH, data[:1024], 0)
    c1 = oracle.chunk_cv(kw, oracle.KEYED_HASH, data[1024:], 1)
    root = oracle.compress(kw, c0 + c1, 0, 64, oracle.KEYED_HASH | oracle.PARENT | oracle.ROOT)[:8]
    assert oracle.hash(data, key) == struct.pack("<8I", *root)
    # the second chunk's counter is its index: counter 0 for it changes the digest
    c1_wrong = oracle.chunk_cv(kw, oracle.KEYED_HASH, data[1024:], 0)
    wrong = oracle.compress(kw, c0 + c1_wrong, 0, 64, oracle.KEYED_HASH | oracle.PARENT | oracle.ROOT)[:8]
    assert struct.pack("<8I", *wrong) != oracle.hash(data, key)


def test_empty_input_is_one_zero_block_of_length_zero():
    for key in (None, _rng_bytes(41, 32)):
        kw = _key_words(key) if key else oracle.iv()
        mode = oracle.KEYED_HASH if key else 0
        out = oracle.compress(kw, [0] * 16, 0, 0, mode | oracle.CHUNK_START | oracle.CHUNK_END | oracle.ROOT)
        assert oracle.hash(b"", key) == struct.pack("<8I", *out[:8])


def test_keyed_differs_from_default_and_flips_propagate():
    data = bytearray(_rng_bytes(51, 5000))
    key = bytearray(_rng_bytes(52, 32))
    base = oracle.hash(bytes(data), bytes(key))
    assert base != oracle.hash(bytes(data))
    for pos in (0, 1023, 1024, 4999):
        d2 = bytearray(data)
        d2[pos] ^= 0x01
        assert oracle.hash(bytes(d2), bytes(key)) != base
    for pos in (0, 31):
        k2 = bytearray(key)
        k2[pos] ^= 0x80
        assert oracle.hash(bytes(data), bytes(k2)) != base
    # a trailing zero byte is not padding: length is part of the hash
    assert oracle.hash(bytes(data) + b"\0", bytes(key)) != base


def test_subtree_cvs_compose_to_the_hash():
    # a 3-way split 4096 + 2048 + 37 chunks of one input, each hashed as a subtree with its
    # counter offset, reassembled by the tree rule, gives the whole-input digest
    key = _rng_bytes(61, 32)
    kw = _key_words(key)
    data = _rng_bytes(62, 6181 * 1024 - 5)
    a = oracle.subtree_cv(data[:4096 * 1024], 0, key)
    b = oracle.subtree_cv(data[4096 * 1024:6144 * 1024], 4096, key)
    c = oracle.subtree_cv(data[6144 * 1024:], 6144, key)
    root = oracle.parent_cv(kw, oracle.KEYED_HASH, a, oracle.parent_cv(kw, oracle.KEYED_HASH, b, c), is_root=True)
    assert struct.pack("<8I", *root) == oracle.hash(data, key)
    # the counter offset matters
    assert oracle.subtree_cv(data[4096 * 1024:6144 * 1024], 0, key) != b
