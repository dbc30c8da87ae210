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
    # message ends split in pass 0 (a last group of more than half a workgroup that is not a
    # power of two): 456 chunks at one chunk per lane, 813 at two, 1725 at one and at four
    [456 * 1024 + 7, 813 * 1024, 1725 * 1024 + 11, 3000],
    [70100 * 1024 - 100],  # split end, then a pair node in a pass that is not the last
]


@pytest.fixture(params=[1, 2, 4])
def chunks_per_lane(request, monkeypatch):
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", str(request.param))
    return request.param


@pytest.mark.parametrize("lengths", LENGTH_SETS)
def test_plan_invariants(lengths, chunks_per_lane):
    splits = _check_plan(lengths, chunks_per_lane)
    if lengths == LENGTH_SETS[-2]:
        assert splits >= 1, "this set splits a message end at every chunks-per-lane setting"


def _check_plan(lengths, chunks_per_lane):
    """Asserts the plan's structural invariants; returns the number of split message ends."""
    plan = b3.debug_plan_batch(lengths)
    n = len(lengths)
    finals = [0] * n
    units = {i: _chunks(int(L)) for i, L in enumerate(lengths)}  # chunks (pass 0) or nodes entering the pass
    inputs = {}  # message -> the input CV indices of its nodes' subtrees, in tree order
    splits = 0
    for pi, p in enumerate(plan):
        lanes = p["lanes"]
        per_node = chunks_per_lane if pi == 0 else 1
        assert lanes == 256 and p["chunks_per_lane"] == per_node
        span = lanes * per_node
        by_msg = {}
        out_seen = set()
        first_idx = p["wg_first_seg"]
        for w in range(len(p["wg_levels"])):
            segs = p["segs"][first_idx[w]:first_idx[w + 1]]
            assert segs, "every workgroup holds a segment"
            used = 0
            for (msg, first, dst, lane, count, final, pair) in segs:
                assert 1 <= count <= lanes
                assert lane % _next_pow2(count) == 0, "segment not aligned to its power of two"
                assert lane >= used and lane + count <= lanes, "segments overlap or overflow"
                used = lane + count
                by_msg.setdefault(msg, []).append((first, count, dst, final, pair))
                if final:
                    finals[msg] += 1
                else:
                    assert dst not in out_seen and dst < p["out_cvs"]
                    out_seen.add(dst)
            assert p["wg_levels"][w] == max(_ceil_log2(s[4]) for s in segs)
        assert len(out_seen) == p["out_cvs"]
        next_inputs = {}
        for msg, spans in by_msg.items():
            spans.sort()
            if pi == 0:
                # aligned groups of `span` chunks from chunk 0; the last may be split into its
                # left subtree (the largest power of two below its node count) and the rest
                assert not any(sp[4] for sp in spans), "no pair nodes in pass 0"
                k_groups = (units[msg] + span - 1) // span
                assert len(spans) in (k_groups, k_groups + 1)
                for k in range(k_groups - 1):
                    assert spans[k][0] == k * span and spans[k][1] == span // per_node
                tail_units = units[msg] - (k_groups - 1) * span
                tail_nodes = (tail_units + per_node - 1) // per_node
                if len(spans) == k_groups + 1:
                    splits += 1
                    (fa, ca, _, _, _), (fb, cb, _, _, _) = spans[-2:]
                    assert k_groups > 1, "a message's only group is never split"
                    assert 2 * tail_nodes > lanes and tail_nodes & (tail_nodes - 1)
                    assert ca == 1 << (tail_nodes.bit_length() - 1) and ca + cb == tail_nodes
                    assert fa == (k_groups - 1) * span and fb == fa + ca * per_node
                else:
                    assert spans[-1][0] == (k_groups - 1) * span and spans[-1][1] == tail_nodes
            else:
                # nodes in aligned groups of `span`; a pair node only at the message's end,
                # reading the two CVs its pass-0 split produced
                nodes = inputs[msg]
                for k, (first, count, dst, final, pair) in enumerate(spans):
                    got = [[first + x] for x in range(count)]
                    if pair:
                        assert k == len(spans) - 1
                        got[-1] = [first + count - 1, first + count]
                    assert got == nodes[k * span:k * span + count]
                assert sum(sp[1] for sp in spans) == len(nodes)
            if not spans[0][3]:
                # CVs of this pass in tree order; a split end's two CVs form one next node
                dsts = [sp[2] for sp in spans]
                if pi == 0 and len(spans) == (units[msg] + span - 1) // span + 1:
                    next_inputs[msg] = [[d] for d in dsts[:-2]] + [dsts[-2:]]
                else:
                    next_inputs[msg] = [[d] for d in dsts]
                assert [d for ds in next_inputs[msg] for d in ds] == list(range(dsts[0], dsts[0] + len(dsts)))
        units = {msg: len(v) for msg, v in next_inputs.items()}
        inputs = next_inputs
    assert finals == [1] * n, "every message is finished exactly once"
    return splits


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
        K = p["chunks_per_lane"]
        for (msg, first, dst, lane, count, final, pair) in p["segs"]:
            kw = list(struct.unpack("<8I", keys[msg])) if keys else oracle.iv()
            mode = oracle.KEYED_HASH if keys else 0
            if pi == 0:
                # each lane folds its run of K chunks into one node, then the nodes pair up
                o, L = offsets[msg], lengths[msg]
                msg_bytes = data[o:o + L]
                n_msg = _chunks(L)
                nodes = []
                for x in range(count):
                    c0 = first + x * K
                    run = range(c0, min(c0 + K, n_msg))
                    lone = final and count == 1
                    cvs = [oracle.chunk_cv(kw, mode, msg_bytes[1024 * j:1024 * (j + 1)], j,
                                           is_root=lone and len(run) == 1) for j in run]
                    nodes.append(_pair_reduce(cvs, kw, mode, lone))
            else:
                nodes = cvs_in[first:first + count]
                if pair:
                    # the two subtrees of a message end split in pass 0
                    nodes[-1] = oracle.parent_cv(kw, mode, cvs_in[first + count - 1], cvs_in[first + count],
                                                 is_root=False)
            top = _pair_reduce(nodes, kw, mode, final)
            if final:
                digests[msg] = struct.pack("<8I", *top)
            else:
                cvs_out[dst] = top
        cvs_in = cvs_out
    return digests


@pytest.mark.parametrize("keyed", [False, True])
def test_executed_plan_matches_oracle(keyed, chunks_per_lane):
    rng = np.random.Generator(np.random.PCG64(11))
    lengths = [0, 1, 63, 64, 65, 1023, 1024, 1025, 13 * 1024 + 17, 3 * 1024 + 1000, 65 * 1024 + 5,
               256 * 1024, 256 * 1024 + 1, 511 * 1024 + 9, 456 * 1024 + 7, 813 * 1024, 1725 * 1024 + 11] + \
        rng.integers(0, 300 * 1024, size=12).tolist()
    offsets, pos = [], 0
    for L in lengths:
        offsets.append(pos)
        pos += (L + 31) // 16 * 16
    data = rng.bytes(pos)
    keys = [rng.bytes(32) for _ in lengths] if keyed else None
    got = _execute_plan(data, offsets, lengths, keys)
    for i, (o, L) in enumerate(zip(offsets, lengths)):
        assert got[i] == oracle.hash(data[o:o + L], keys[i] if keys else None), (i, L)


def test_executed_plan_deep_tree(monkeypatch):
    # 70,000 chunks of one message at one chunk per lane: pass 0 (274 groups) ->
    # pass 1 (2 groups) -> pass 2
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", "1")
    rng = np.random.Generator(np.random.PCG64(12))
    L = 70000 * 1024 - 100
    data = rng.bytes(L)
    key = rng.bytes(32)
    plan = b3.debug_plan_batch([L])
    assert len(plan) == 3
    assert _execute_plan(data, [0], [L], [key])[0] == oracle.hash(data, key)


def test_executed_plan_split_end_deep_tree(monkeypatch):
    # 70,100 chunks at one chunk per lane: the last group (212 chunks) is split into 128 + 84
    # in pass 0; pass 1 has 274 nodes, the last a pair, in two groups; pass 2 finishes
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", "1")
    rng = np.random.Generator(np.random.PCG64(13))
    L = 70100 * 1024 - 100
    data = rng.bytes(L)
    plan = b3.debug_plan_batch([L])
    assert len(plan) == 3
    assert [s[4] for s in plan[0]["segs"] if s[4] != 256] == [128, 84]
    assert [s[6] for s in plan[1]["segs"]] == [False, True]
    assert _execute_plan(data, [0], [L], None)[0] == oracle.hash(data)


def test_chunks_per_lane_choice(monkeypatch):
    monkeypatch.delenv("BLAKE3_GPU_CHUNKS_PER_LANE", raising=False)
    ks = [b3.debug_plan_batch([size])[0]["chunks_per_lane"] for size in
          (1 << 20, 256 << 20, 1 << 30, 2 << 30, 4 << 30, 16 << 30)]
    assert ks[0] == 1 and ks[-1] == 4 and ks == sorted(ks), ks
    assert all(k in (1, 2, 4) for k in ks)
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", "2")
    assert b3.debug_plan_batch([1 << 20])[0]["chunks_per_lane"] == 2


# ---- property-based sweep: random mixes of lengths --------------------------------------
#
# Lengths near chunk and workgroup boundaries, small and large, in random mixes; seeded
# (derandomized) so that every run checks the same cases, and with no example database
# written to disk.

from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

_NEAR = st.sampled_from([1024, 64 * 1024, 128 * 1024, 256 * 1024, 512 * 1024, 1024 * 1024])


def _length(max_bytes):
    return st.one_of(
        st.integers(0, 4096),
        st.builds(lambda b, k, d: max(0, min(max_bytes, b * k + d)), _NEAR, st.integers(1, 8),
                  st.sampled_from([-1, 0, 1, 17])),
        st.integers(0, max_bytes),
    )


_SWEEP = settings(max_examples=120, derandomize=True, database=None, deadline=None,
                  suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


@_SWEEP
@given(lengths=st.lists(_length(96 * 1024 * 1024), min_size=1, max_size=300),
       k=st.sampled_from([1, 2, 4]))
def test_plan_invariants_on_random_mixes(lengths, k, monkeypatch):
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", str(k))
    _check_plan(lengths, k)


@settings(max_examples=25, derandomize=True, database=None, deadline=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(lengths=st.lists(_length(1100 * 1024), min_size=1, max_size=12),
       k=st.sampled_from([1, 2, 4]), keyed=st.booleans(), seed=st.integers(0, 2**32 - 1))
def test_executed_plan_matches_oracle_on_random_mixes(lengths, k, keyed, seed, monkeypatch):
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", str(k))
    rng = np.random.Generator(np.random.PCG64(seed))
    offsets, pos = [], 0
    for L in lengths:
        offsets.append(pos)
        pos += (L + 31) // 16 * 16
    data = rng.bytes(pos)
    keys = [rng.bytes(32) for _ in lengths] if keyed else None
    got = _execute_plan(data, offsets, lengths, keys)
    for i, (o, L) in enumerate(zip(offsets, lengths)):
        assert got[i] == oracle.hash(data[o:o + L], keys[i] if keys else None), (i, L)


def test_a_pass_beyond_one_launch_is_too_big(monkeypatch):
    # five messages of 2^42 bytes at four chunks per lane: 5 * 2^22 leaf workgroups of 256
    # lanes, more than the 2^32 - 1 work-items of one launch (refused before any table is built)
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", "4")
    with pytest.raises(b3.Blake3GpuError) as err:
        b3.debug_plan_batch([1 << 42] * 5)
    assert err.value.status == b3.ETOOBIG
