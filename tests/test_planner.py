"""The batch planner (host logic, no GPU).

Structural invariants of the launch plan, and an execution of the plan on the CPU with
the oracle's chunk and parent primitives, reducing every segment with the workgroups'
pairing rule (pair neighbours, carry an odd last node up unchanged). That the executed
plan reproduces the oracle's digests shows, independently of any GPU, that the grouping
into aligned segments plus the pairing rule builds the BLAKE3 tree.
"""
import struct

import numpy as np
import pytest

import blake3_merkle_tree_amd as b3
import oracle


def _chunks(n):
    return 1 if n == 0 else (n + 1023) // 1024


def _next_pow2(n):
    r = 1
    while r < n:
        r *= 2
    return r


def _ceil_log2(n):
    return (n - 1).bit_length() if n > 1 else 0


LENGTH_SETS = [
    [0],
    [1],
    [1024],
    [1025],
    [256 * 1024],
    [256 * 1024 + 1],
    [300 * 1024 + 5, 0, 1, 5000, 64 * 1024, 64 * 1024],
    [64 * 1024] * 37,
    [1024 * 1024 + 1] + [17] * 300,
    list(np.random.Generator(np.random.PCG64(3)).integers(0, 600 * 1024, size=60)),
    [65 * 1024 * 1024 + 3, 2048],  # three passes for the first message
]


@pytest.mark.parametrize("lengths", LENGTH_SETS)
def test_plan_invariants(lengths):
    plan = b3.debug_plan_batch(lengths)
    n = len(lengths)
    finals = [0] * n
    nodes = {i: _chunks(L) for i, L in enumerate(lengths)}  # nodes entering the pass
    for pi, p in enumerate(plan):
        lanes = p["lanes"]
        assert lanes == 256
        covered = {}
        out_seen = set()
        first_idx = p["wg_first_seg"]
        for w in range(len(p["wg_levels"])):
            segs = p["segs"][first_idx[w]:first_idx[w + 1]]
            assert segs, "every workgroup holds a segment"
            used = 0
            for (msg, first, dst, lane, count, final) in segs:
                assert 1 <= count <= lanes
                assert lane % _next_pow2(count) == 0, "segment not aligned to its power of two"
                assert lane >= used and lane + count <= lanes, "segments overlap or overflow"
                used = lane + count
                covered.setdefault(msg, []).append((first, count))
                if final:
                    finals[msg] += 1
                else:
                    assert dst not in out_seen and dst < p["out_cvs"]
                    out_seen.add(dst)
            assert p["wg_levels"][w] == max(_ceil_log2(s[4]) for s in segs)
        assert len(out_seen) == p["out_cvs"]
        # each message still open is covered exactly once, in aligned groups of `lanes`
        for msg, spans in covered.items():
            spans.sort()
            total = sum(c for _, c in spans)
            assert total == nodes[msg]
            base = spans[0][0]
            for k, (first, count) in enumerate(spans):
                assert first == base + k * lanes
            if pi == 0:
                assert base == 0
        nodes = {msg: len(spans) for msg, spans in covered.items() if len(spans) > 1}
    assert finals == [1] * n, "every message is finished exactly once"


def _pair_reduce(nodes, kw, mode, final):
    while len(nodes) > 1:
        nxt = []
        for i in range(0, len(nodes) - 1, 2):
            top = final and len(nodes) == 2
            nxt.append(oracle.parent_cv(kw, mode, nodes[i], nodes[i + 1], is_root=top))
        if len(nodes) % 2:
            nxt.append(nodes[-1])
        nodes = nxt
    return nodes[0]


def _execute_plan(data, offsets, lengths, keys):
    plan = b3.debug_plan_batch(lengths)
    digests = [None] * len(lengths)
    cvs_in = []
    for pi, p in enumerate(plan):
        cvs_out = [None] * p["out_cvs"]
        for (msg, first, dst, lane, count, final) in p["segs"]:
            kw = list(struct.unpack("<8I", keys[msg])) if keys else oracle.iv()
            mode = oracle.KEYED_HASH if keys else 0
            if pi == 0:
                o, L = offsets[msg], lengths[msg]
                msg_bytes = data[o:o + L]
                nodes = [oracle.chunk_cv(kw, mode, msg_bytes[1024 * j:1024 * (j + 1)], j,
                                         is_root=final and count == 1)
                         for j in range(first, first + count)]
            else:
                nodes = cvs_in[first:first + count]
            top = _pair_reduce(nodes, kw, mode, final)
            if final:
                digests[msg] = struct.pack("<8I", *top)
            else:
                cvs_out[dst] = top
        cvs_in = cvs_out
    return digests


@pytest.mark.parametrize("keyed", [False, True])
def test_executed_plan_matches_oracle(keyed):
    rng = np.random.Generator(np.random.PCG64(11))
    lengths = [0, 1, 63, 64, 65, 1023, 1024, 1025, 13 * 1024 + 17, 3 * 1024 + 1000, 65 * 1024 + 5,
               256 * 1024, 256 * 1024 + 1, 511 * 1024 + 9] + rng.integers(0, 300 * 1024, size=12).tolist()
    offsets, pos = [], 0
    for L in lengths:
        offsets.append(pos)
        pos += (L + 31) // 16 * 16
    data = rng.bytes(pos)
    keys = [rng.bytes(32) for _ in lengths] if keyed else None
    got = _execute_plan(data, offsets, lengths, keys)
    for i, (o, L) in enumerate(zip(offsets, lengths)):
        assert got[i] == oracle.hash(data[o:o + L], keys[i] if keys else None), (i, L)


def test_executed_plan_deep_tree():
    # 70,000 chunks of one message: pass 0 (274 groups) -> pass 1 (2 groups) -> pass 2
    rng = np.random.Generator(np.random.PCG64(12))
    L = 70000 * 1024 - 100
    data = rng.bytes(L)
    key = rng.bytes(32)
    plan = b3.debug_plan_batch([L])
    assert len(plan) == 3
    assert _execute_plan(data, [0], [L], [key])[0] == oracle.hash(data, key)
