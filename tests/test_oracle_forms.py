"""Internal consistency of the oracle's four forms (CPU only).

The recursive (top-down) definition, the stack-merge incremental hasher, the same hasher
fed in arbitrary pieces, and the multi-threaded aligned-group form must agree bit for bit.
A mistake in any one form (a wrong split, a merge at the wrong time, a chunk closed too
early so that a lone chunk misses ROOT, a group boundary off by one) breaks one of them.
"""
import numpy as np
import pytest

import oracle


def _bytes(seed, n):
    return np.random.Generator(np.random.PCG64(seed)).bytes(n)


TAILS = [1, 63, 64, 65, 1023, 1024]


@pytest.mark.parametrize("keyed", [False, True])
def test_recursive_equals_stack_merge_all_small_trees(keyed):
    key = _bytes(7, 32) if keyed else None
    data = _bytes(8, 130 * 1024)
    assert oracle.hash(b"", key) == oracle.hash_recursive(b"", key)
    for n in range(1, 131):
        for t in TAILS:
            L = (n - 1) * 1024 + t
            assert oracle.hash(data[:L], key) == oracle.hash_recursive(data[:L], key), (n, t)


def test_incremental_split_points():
    rng = np.random.Generator(np.random.PCG64(9))
    key = _bytes(10, 32)
    data = _bytes(11, 40 * 1024 + 333)
    ref = oracle.hash(data, key)
    # one byte at a time over a short prefix, then the rest
    h = oracle.Hasher(key)
    for i in range(3000):
        h.update(data[i:i + 1])
    h.update(data[3000:])
    assert h.digest() == ref
    # splits exactly on block and chunk boundaries
    for step in (64, 1024, 2048, 4096):
        h = oracle.Hasher(key)
        for i in range(0, len(data), step):
            h.update(data[i:i + step])
        assert h.digest() == ref
    # random split points
    for _ in range(20):
        cuts = sorted(rng.integers(0, len(data), size=int(rng.integers(1, 12))).tolist())
        h = oracle.Hasher(key)
        prev = 0
        for c in cuts + [len(data)]:
            h.update(data[prev:c])
            prev = c
        assert h.digest() == ref
    # finalize does not consume state: a prefix digest, then more input
    h = oracle.Hasher(key)
    h.update(data[:5000])
    assert h.digest() == oracle.hash(data[:5000], key)
    h.update(data[5000:])
    assert h.digest() == ref


@pytest.mark.parametrize("nthreads", [1, 2, 3, 8])
def test_multithreaded_equals_single_threaded(nthreads):
    key = _bytes(12, 32)
    data = _bytes(13, 3 * 1024 * 1024 + 777)
    for L in (0, 1, 1024, 1025, 64 * 1024, 257 * 1024 + 5, 1024 * 1024, len(data)):
        assert oracle.hash_mt(data[:L], key, nthreads) == oracle.hash(data[:L], key), L
        assert oracle.hash_mt(data[:L], None, nthreads) == oracle.hash(data[:L]), L


def test_batch_equals_individual_hashes():
    rng = np.random.Generator(np.random.PCG64(14))
    lens = [0, 1, 63, 64, 65, 1023, 1024, 1025, 5000] + rng.integers(0, 70000, size=20).tolist()
    offs, pos = [], 0
    for L in lens:
        offs.append(pos)
        pos += (L + 15) // 16 * 16 + 16
    base = _bytes(15, pos)
    keys = _bytes(16, 32 * len(lens))
    got = oracle.hash_batch(base, offs, lens, keys, nthreads=4)
    for i, (o, L) in enumerate(zip(offs, lens)):
        assert got[i] == oracle.hash(base[o:o + L], keys[32 * i:32 * i + 32])
    got_plain = oracle.hash_batch(base, offs, lens, None, nthreads=3)
    for i, (o, L) in enumerate(zip(offs, lens)):
        assert got_plain[i] == oracle.hash(base[o:o + L])
