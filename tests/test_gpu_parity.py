"""GPU parity: every digest of the HIP path equals the CPU oracle's, bit for bit.

The HIP path is called through the C ABI (via the thin binding); the oracle hashes a host
copy of the same device bytes. Cases: brute force over chunk counts and tail lengths
(partial blocks, single-chunk roots, non-power-of-two trees, workgroup and level
boundaries), the empty input, misaligned views, non-default streams, batches with gap
bytes of 0xA5 between messages (an over-read changes the digest), split message ends and
seeded random batches, every workload at full size in the launch configuration the
benchmark times, single messages just above one round whose excess runs on quads in the
same launch, extended output and subtree CVs (share roots of a 4 GiB and a 256 MiB
input, hashed separately with their chunk bases, combine to the digest), and the library's
scratch: a forced allocation failure, scratch of arbitrary prior contents, repeated runs,
and calls shared between streams, host threads and a stream held behind long work; and graph
capture (replays equal eager results; a table-planned batch is refused under capture).
"""
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TAILS = [1, 63, 64, 65, 1023, 1024]
NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def b3():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import blake3_merkle_tree_amd as mod
    return mod


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _host(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.uint8).reshape(-1).cpu().numpy()


def _digests_to_bytes(d):
    return [bytes(row) for row in d.cpu().numpy().reshape(-1, 32)]


def _say(*a):
    print(*a, flush=True)


# BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS: inputs up to this many chunks take the quad leaf
# (four lanes per chunk); "0" sends every input to the lane-per-chunk leaf
QUAD_OFF, QUAD_ALL = "0", str(1 << 62)


@pytest.mark.parametrize("quad", ["default", QUAD_OFF])
def test_brute_force_lengths_single_call(b3, dev, monkeypatch, quad):
    if quad != "default":
        monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", quad)
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(400 * 1024, 21, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(22)[0].tolist())
    lengths = [0] + [(n - 1) * 1024 + t for n in range(1, 301) for t in TAILS] + \
              [(n - 1) * 1024 + t for n in (384, 399, 400) for t in (1, 1024)]
    for keyed in (True, False):
        _say("brute force single-call, keyed =", keyed, "cases", len(lengths))
        outs = torch.empty((len(lengths), 32), dtype=torch.uint8, device=dev)
        for i, L in enumerate(lengths):
            if keyed:
                b3.keyed_hash(buf[:L], key, out=outs[i])
            else:
                b3.hash(buf[:L], out=outs[i])
        got = _digests_to_bytes(outs)
        want = oracle.hash_batch(host, [0] * len(lengths), lengths,
                                 key * len(lengths) if keyed else None, nthreads=NTHREADS)
        bad = [L for L, g, w in zip(lengths, got, want) if g != w]
        assert not bad, f"{len(bad)} lengths differ, first {bad[:5]}"


@pytest.mark.parametrize("quad", ["default", QUAD_OFF])
def test_every_tail_length(b3, dev, monkeypatch, quad):
    # every length of a message's last chunk, 0..1024 bytes, after 0, 1 and 4 full chunks:
    # the last chunk's final block, and within it the 16-byte piece that holds the last
    # byte, take every position; single calls and one batch with 0xA5 gaps
    if quad != "default":
        monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", quad)
    from blake3_merkle_tree_amd import workloads
    lengths = [0] + [full * 1024 + t for full in (0, 1, 4) for t in range(1, 1025)]
    offs, total = workloads.pack_messages(lengths)
    base = torch.full((total,), 0xA5, dtype=torch.uint8, device=dev)
    data = workloads.random_bytes(total, 34, dev)
    for o, L in zip(offs, lengths):
        base[o:o + L] = data[o:o + L]
    host = _host(base)
    keys = workloads.key_bytes(35, len(lengths))
    want = oracle.hash_batch(host, offs, lengths, keys.numpy().tobytes(), nthreads=NTHREADS)
    _say("every tail length, single calls, cases", len(lengths))
    outs = torch.empty((len(lengths), 32), dtype=torch.uint8, device=dev)
    for i, (o, L) in enumerate(zip(offs, lengths)):
        b3.keyed_hash(base[o:o + L], bytes(keys[i].tolist()), out=outs[i])
    got = _digests_to_bytes(outs)
    bad = [L for L, g, w in zip(lengths, got, want) if g != w]
    assert not bad, f"{len(bad)} lengths differ, first {bad[:5]}"
    _say("every tail length, one batch")
    got = _digests_to_bytes(b3.keyed_hash_batch(base, offs, lengths, keys.to(dev)))
    bad = [L for L, g, w in zip(lengths, got, want) if g != w]
    assert not bad, f"{len(bad)} lengths differ in the batch, first {bad[:5]}"


@pytest.mark.parametrize("quad,fused", [("default", "1"), (QUAD_ALL, "1"), ("default", "0"), (QUAD_ALL, "0")])
def test_level_boundaries(b3, dev, monkeypatch, quad, fused):
    # 256-chunk leaf workgroups and 256-CV level workgroups: counts around 256 and 256^2;
    # with the quad leaf, 64-chunk workgroups: counts around 64, 64*256 and 64*256^2.
    # 200,000, 262,144 and 262,145 chunks leave 782, 1024 and 1025 leaf CVs: the first
    # level pass ends with 4, 4 and 5 CVs. 25,600, 60,000 and 91,137 chunks give level groups
    # of 100, 235, and 256 + 101 CVs (quad leaf: 256 + 144, 256 * 3 + 170, 256 * 5 + 145),
    # so level trees whose widest level has 33-64 and 65-128 output positions.
    # fused: level passes run inside the leaf launch (last-arrival tickets), or as
    # separate level launches
    if quad != "default":
        monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", quad)
    monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", fused)
    from blake3_merkle_tree_amd import workloads
    chunks = [63, 64, 65, 255, 256, 257, 511, 512, 513, 16383, 16384, 16385, 25600, 32767, 32768, 32769, 60000,
              65535, 65536, 65537,
              91137, 131073, 200000, 262144, 262145]
    buf = workloads.random_bytes(262145 * 1024, 23, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(24)[0].tolist())
    lengths = [(n - 1) * 1024 + t for n in chunks for t in (1, 1000, 1024)]
    _say("level boundaries", len(lengths), "cases")
    outs = torch.empty((len(lengths), 32), dtype=torch.uint8, device=dev)
    for i, L in enumerate(lengths):
        b3.keyed_hash(buf[:L], key, out=outs[i])
    want = oracle.hash_batch(host, [0] * len(lengths), lengths, key * len(lengths), nthreads=NTHREADS)
    assert _digests_to_bytes(outs) == want


@pytest.mark.parametrize("split", ["1", "0"])
def test_one_round_and_a_quad_tail(b3, dev, monkeypatch, split):
    # a message just above 2^16, 2^17 or 2^18 chunks hashes its first 2^16 (2^17, 2^18) chunks
    # as one round of 256 leaf workgroups at one (two, four) chunks per lane and the tail past
    # them, up to 2^15 chunks, on quad workgroups in the same launch; both subtrees and their
    # parent in one more launch (up to 256 tail CVs in a 512-lane tree, more in a 1024-lane
    # one). Lengths around both ends of the three ranges and across 2^14 tail chunks, keyed and
    # default mode; with BLAKE3_GPU_SPLIT_TAIL=0 the same lengths take the ordinary leaf.
    monkeypatch.setenv("BLAKE3_GPU_SPLIT_TAIL", split)
    from blake3_merkle_tree_amd import workloads
    k16, k17, k18 = (1 << 16) * 1024, (1 << 17) * 1024, (1 << 18) * 1024
    lengths = [k16 + 1, k16 + 3000, k16 + (16 << 20), k16 + (16 << 20) + 1, k16 + (32 << 20), k16 + (32 << 20) + 1,
               k17 + 1, k17 + 1024, k17 + 1025, k17 + 64 * 1024, k17 + 64 * 1024 + 1, k17 + (8 << 20),
               k17 + (16 << 20), k17 + (16 << 20) + 1, k17 + (24 << 20) + 5, k17 + (32 << 20) + 1,
               k18 + 1, k18 + 777, k18 + (64 << 10) + 5, k18 + (16 << 20) - 3, k18 + (16 << 20),
               k18 + (16 << 20) + 1, k18 + (32 << 20), k18 + (32 << 20) + 1]
    buf = workloads.random_bytes(max(lengths), 25, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(26)[0].tolist())
    _say("one round and a quad tail", len(lengths), "lengths, split", split)
    outs = torch.empty((len(lengths), 32), dtype=torch.uint8, device=dev)
    for i, L in enumerate(lengths):
        b3.keyed_hash(buf[:L], key, out=outs[i])
    want = oracle.hash_batch(host, [0] * len(lengths), lengths, key * len(lengths), nthreads=NTHREADS)
    assert _digests_to_bytes(outs) == want
    for L in (k17 + 1025, k18 + 777):
        assert bytes(b3.hash(buf[:L]).cpu().tolist()) == oracle.hash_mt(host[:L], None, NTHREADS), L


def test_random_single_sizes(b3, dev):
    # seeded sizes, 12 spread log-uniformly from 1 B to 300 MiB and 28 uniformly from 32 MiB to
    # 300 MiB, so that every leaf form meets arbitrary lengths: the quad leaf, one, two and
    # four chunks per lane picked by the busiest-CU rule, and the split just above a round
    from blake3_merkle_tree_amd import workloads
    rng = np.random.default_rng(31)
    lengths = sorted([int(x) for x in np.exp(rng.uniform(0.0, np.log(300 << 20), 12))] +
                     [int(x) for x in rng.integers(32 << 20, 300 << 20, 28)])
    buf = workloads.random_bytes(max(lengths), 32, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(33)[0].tolist())
    _say("random single sizes", lengths[:3], "...", lengths[-3:])
    outs = torch.empty((len(lengths), 32), dtype=torch.uint8, device=dev)
    for i, L in enumerate(lengths):
        b3.keyed_hash(buf[:L], key, out=outs[i])
    want = oracle.hash_batch(host, [0] * len(lengths), lengths, key * len(lengths), nthreads=NTHREADS)
    assert _digests_to_bytes(outs) == want


def test_quad_tail_subtree_cv_and_xof(b3, dev):
    # the same split with root_flag 0: a subtree CV at a chunk base, and the extended output of
    # a message whose right subtree (2^17 + 100 chunks) takes it
    from blake3_merkle_tree_amd import workloads
    L = ((1 << 18) + (1 << 17) + 100) * 1024 - 9
    buf = workloads.random_bytes(L, 27, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(28)[0].tolist())
    S = (1 << 17) * 1024 + 3000
    base = 1 << 20
    _say("quad tail subtree cv", S, "bytes, chunk base", base)
    got = b3.subtree_cv(buf[:S], key, chunk_base=base).cpu().numpy().view(np.uint32).tolist()
    assert got == oracle.subtree_cv(host[:S].tobytes(), base, key)
    _say("quad tail xof", L, "bytes")
    got = bytes(b3.hash_xof(buf, key, out_len=200).cpu().tolist())
    assert got == oracle.hash_xof(host.tobytes(), key, out_len=200)


def test_empty_and_dtypes_and_misaligned_views(b3, dev):
    from blake3_merkle_tree_amd import workloads
    key = bytes(workloads.key_bytes(25)[0].tolist())
    empty = torch.empty(0, dtype=torch.uint8, device=dev)
    assert bytes(b3.hash(empty).cpu().tolist()) == oracle.hash(b"")
    assert bytes(b3.keyed_hash(empty, key).cpu().tolist()) == oracle.hash(b"", key)
    buf = workloads.random_bytes(70000, 26, dev)
    host = _host(buf)
    for start in (1, 3, 8, 15, 16):  # views not 16-byte aligned are re-allocated by the binding
        got = bytes(b3.keyed_hash(buf[start:], key).cpu().tolist())
        assert got == oracle.hash(host[start:].tobytes(), key), start
    f = torch.randn(3, 1000, 7, dtype=torch.float32, device=dev)
    assert bytes(b3.keyed_hash(f, key).cpu().tolist()) == oracle.hash(_host(f).tobytes(), key)
    ft = f.transpose(0, 2)  # non-contiguous: hashed as its contiguous copy
    assert bytes(b3.hash(ft).cpu().tolist()) == oracle.hash(_host(ft.contiguous()).tobytes())


def test_non_default_stream(b3, dev):
    from blake3_merkle_tree_amd import workloads
    key = bytes(workloads.key_bytes(27)[0].tolist())
    s = torch.cuda.Stream(device=dev)
    buf = workloads.random_bytes(3 * 1024 * 1024 + 7, 28, dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = b3.keyed_hash(buf, key)
    s.synchronize()
    assert bytes(out.cpu().tolist()) == oracle.hash(_host(buf).tobytes(), key)


def test_batch_mixed_lengths_with_gaps(b3, dev):
    from blake3_merkle_tree_amd import workloads
    rng = np.random.Generator(np.random.PCG64(29))
    lengths = [0, 1, 63, 64, 65, 1023, 1024, 1025, 5000, 64 * 1024, 256 * 1024, 256 * 1024 + 1,
               300 * 1024 + 5] + rng.integers(0, 400 * 1024, size=100).tolist() + [1] * 50
    offs, total = workloads.pack_messages(lengths)
    base = torch.full((total,), 0xA5, dtype=torch.uint8, device=dev)
    data = workloads.random_bytes(total, 30, dev)
    for o, L in zip(offs, lengths):
        base[o:o + L] = data[o:o + L]
    host = _host(base)
    keys = workloads.key_bytes(31, len(lengths))
    for keyed in (True, False):
        _say("batch mixed, keyed =", keyed)
        out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev) if keyed else None)
        want = oracle.hash_batch(host, offs, lengths, keys.numpy().tobytes() if keyed else None,
                                 nthreads=NTHREADS)
        assert _digests_to_bytes(out) == want
    # the batch equals one call per message
    singles = [bytes(b3.keyed_hash(base[o:o + L], bytes(keys[i].tolist())).cpu().tolist())
               for i, (o, L) in enumerate(zip(offs, lengths))]
    assert singles == _digests_to_bytes(b3.keyed_hash_batch(base, offs, lengths, keys.to(dev)))


@pytest.mark.parametrize("fused", ["0", "1"])
def test_random_batches_match_oracle(b3, dev, monkeypatch, fused):
    # seeded random batches through the task table: lengths mixing empty, sub-block,
    # chunk-boundary, multi-workgroup and split-end messages, random 16-byte gaps, keyed
    # and default mode, at one, two and four chunks per lane; the first level pass as its
    # own launch and fused into the leaf launch (last arrival of each level segment)
    monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", fused)
    from blake3_merkle_tree_amd import workloads
    rng = np.random.Generator(np.random.PCG64(2024))

    def length():
        kind = rng.integers(0, 6)
        if kind == 0:
            return int(rng.integers(0, 65))
        if kind == 1:
            return int(rng.integers(1, 9)) * 1024 + int(rng.integers(-1, 2))
        if kind == 2:
            return int(rng.integers(0, 64 * 1024))
        if kind == 3:  # a last leaf group of 129..255 chunks after whole groups: split ends
            return (256 * int(rng.integers(1, 3)) + int(rng.integers(129, 256))) * 1024 - int(rng.integers(0, 1024))
        if kind == 4:
            return int(rng.integers(0, 600 * 1024))
        return int(rng.integers(0, 3 << 20))

    for trial in range(12):
        monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", str((1, 2, 4)[trial % 3]))
        n = int(rng.integers(1, 120))
        lengths = [max(0, length()) for _ in range(n)]
        offs, pos = [], 0
        for L in lengths:
            pos += 16 * int(rng.integers(0, 3))  # random gaps
            offs.append(pos)
            pos += (L + 15) // 16 * 16
        base = torch.full((pos + 16,), 0xA5, dtype=torch.uint8, device=dev)
        data = workloads.random_bytes(pos + 16, 70 + trial, dev)
        for o, L in zip(offs, lengths):
            base[o:o + L] = data[o:o + L]
        host = _host(base)
        keyed = trial % 2 == 0
        keys = workloads.key_bytes(90 + trial, n)
        _say("random batch", trial, "messages", n, "bytes", sum(lengths), "keyed", keyed, "fused", fused)
        out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev) if keyed else None)
        want = oracle.hash_batch(host, offs, lengths, keys.numpy().tobytes() if keyed else None, nthreads=NTHREADS)
        assert _digests_to_bytes(out) == want, (trial, n)


@pytest.mark.parametrize("fused", ["0", "1"])
@pytest.mark.parametrize("chunks_per_lane", ["1", "2", "4"])
def test_batch_split_message_ends(b3, dev, monkeypatch, chunks_per_lane, fused):
    # a message's last group of more than half a workgroup that is not a power of two is
    # split in the leaf pass into its left subtree and the rest, whose parent the level
    # pass computes: 456 chunks split at one chunk per lane, 813 at two, 1725 at one and
    # four; 70,100 chunks put the pair node in a level pass that is not the last. Fused:
    # the first level pass (pair nodes included) runs in the leaf launch, a second one after
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", chunks_per_lane)
    monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", fused)
    from blake3_merkle_tree_amd import workloads
    lengths = [456 * 1024 + 7, 813 * 1024, 1725 * 1024 + 11, 3000, 70100 * 1024 - 100, 1, 200 * 1024 + 5]
    plan = b3.debug_plan_batch(lengths)
    assert any(s[6] for p in plan[1:] for s in p["segs"]), "the plan has a split message end"
    offs, total = workloads.pack_messages(lengths)
    base = torch.full((total,), 0xA5, dtype=torch.uint8, device=dev)
    data = workloads.random_bytes(total, 36, dev)
    for o, L in zip(offs, lengths):
        base[o:o + L] = data[o:o + L]
    host = _host(base)
    keys = workloads.key_bytes(37, len(lengths))
    _say("batch split message ends, chunks per lane", chunks_per_lane, "fused", fused)
    out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))
    want = oracle.hash_batch(host, offs, lengths, keys.numpy().tobytes(), nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want
    out = b3.keyed_hash_batch(base, offs, lengths, None)
    want = oracle.hash_batch(host, offs, lengths, None, nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want


@pytest.mark.parametrize("fused", ["0", "1"])
def test_batch_many_level_segments_per_workgroup(b3, dev, monkeypatch, fused):
    # 600 messages of one full 256-chunk group plus an end of 1-7 chunks: the ends pack into
    # a few workgroups dispatched after the 600 full ones, so with the first level pass fused
    # a workgroup is often the last arrival for many two-CV level segments, which it reduces
    # in rounds of up to 64 (slots sized to the largest segment)
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", "1")
    monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", fused)
    from blake3_merkle_tree_amd import workloads
    lengths = [(256 + 1 + i % 7) * 1024 - (i * 37) % 1000 for i in range(600)]
    plan = b3.debug_plan_batch(lengths)
    assert len(plan) == 2 and len(plan[1]["segs"]) == 600
    offs, total = workloads.pack_messages(lengths)
    base = workloads.random_bytes(total, 38, dev)
    host = _host(base)
    keys = workloads.key_bytes(39, len(lengths))
    _say("batch of 600 two-group messages, fused", fused)
    out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))
    want = oracle.hash_batch(host, offs, lengths, keys.numpy().tobytes(), nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want
    out = b3.keyed_hash_batch(base, offs, lengths, None)
    want = oracle.hash_batch(host, offs, lengths, None, nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want


def test_batch_deep_messages(b3, dev):
    # messages with more than 256^2 chunks need a second level pass inside the batch
    from blake3_merkle_tree_amd import workloads
    lengths = [65537 * 1024 + 3, 12, 256 * 1024 * 3 + 17, 0]
    offs, total = workloads.pack_messages(lengths)
    base = workloads.random_bytes(total, 32, dev)
    keys = workloads.key_bytes(33, len(lengths))
    out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))
    want = oracle.hash_batch(_host(base), offs, lengths, keys.numpy().tobytes(), nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want


# ---- workloads at full size -------------------------------------------------------

def _single_workload(b3, dev, name, repeats=1):
    from blake3_merkle_tree_amd import workloads
    t, key = workloads.single(name, dev)
    key = bytes(key.tolist())
    _say(name, "bytes", t.numel() * t.element_size())
    digests = set()
    for _ in range(repeats):
        digests.add(bytes(b3.keyed_hash(t, key).cpu().tolist()))
    assert len(digests) == 1, "repeated runs disagree"
    host = _host(t)
    del t
    torch.cuda.empty_cache()
    want = oracle.hash_mt(host, key, NTHREADS)
    assert digests.pop() == want


def test_workload_mib1(b3, dev):
    _single_workload(b3, dev, "mib1", repeats=3)


def test_workload_fp32_8192(b3, dev):
    _single_workload(b3, dev, "fp32_8192", repeats=2)


def test_workload_gib4(b3, dev, monkeypatch):
    _single_workload(b3, dev, "gib4", repeats=3)
    # the same digest with the level passes fused into the leaf launch, also through the
    # quad leaf (4,194,305 chunks in 65,537 workgroups: three fused levels)
    from blake3_merkle_tree_amd import workloads
    t, key = workloads.single("gib4", dev)
    key = bytes(key.tolist())
    want = bytes(b3.keyed_hash(t, key).cpu().tolist())
    monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", "1")
    assert bytes(b3.keyed_hash(t, key).cpu().tolist()) == want
    monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", QUAD_ALL)
    assert bytes(b3.keyed_hash(t, key).cpu().tolist()) == want


def test_workload_gib16(b3, dev):
    _single_workload(b3, dev, "gib16")


def test_workload_ragged256(b3, dev, monkeypatch):
    # the default plan fuses the first level pass into the leaf launch here; the separate
    # level launch gives the same digests
    from blake3_merkle_tree_amd import workloads
    base, offs, lengths, keys = workloads.ragged_batch(dev)
    assert b3.debug_plan_batch(lengths)[1]["segs"], "the ragged batch has a level pass"
    out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))
    want = oracle.hash_batch(_host(base), offs, lengths, keys.numpy().tobytes(), nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want
    monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", "0")
    assert _digests_to_bytes(b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))) == want


def test_workload_batch64k(b3, dev, monkeypatch):
    from blake3_merkle_tree_amd import workloads
    base, offs, lengths, keys = workloads.uniform_batch(65536, 65536, dev)
    out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))
    again = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))
    assert torch.equal(out, again)
    # the same batch through the launch table agrees
    monkeypatch.setenv("BLAKE3_GPU_BATCH_TABLE", "1")
    assert torch.equal(b3.keyed_hash_batch(base, offs, lengths, keys.to(dev)), out)
    monkeypatch.delenv("BLAKE3_GPU_BATCH_TABLE")
    host = _host(base)
    del base
    want = oracle.hash_batch(host, offs, lengths, keys.numpy().tobytes(), nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want


@pytest.mark.parametrize("staging", ["direct", "lds"])
@pytest.mark.parametrize("group_chunks", [64, 256, 512, 1024])
def test_group_cvs_with_counter_offsets(b3, dev, monkeypatch, group_chunks, staging):
    monkeypatch.setenv("BLAKE3_GPU_STAGING", staging)
    # the leaf pass alone: one CV per aligned group, no ROOT; chunk_base above 2^32
    # exercises the counter's high word; 64-chunk groups run the quad leaf
    from blake3_merkle_tree_amd import workloads
    n_groups = 4
    tail_kib = min(100, group_chunks - 27)  # the last group: a partial one, with a short last chunk
    buf = workloads.random_bytes((n_groups - 1) * group_chunks * 1024 + tail_kib * 1024 + 77, 34, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(35)[0].tolist())
    G = group_chunks * 1024
    for base in (0, group_chunks, (1 << 32) + 2 * group_chunks, (1 << 40) - 4 * group_chunks):
        for keyed in (True, False):
            got = b3.group_cvs(buf, key if keyed else None, chunk_base=base, group_chunks=group_chunks)
            got = got.cpu().numpy().view(np.uint32)
            assert got.shape == (n_groups, 8)
            for g in range(n_groups):
                want = oracle.subtree_cv(host[g * G:(g + 1) * G].tobytes(), base + g * group_chunks,
                                         key if keyed else None)
                assert got[g].tolist() == want, (base, keyed, g)


@pytest.mark.parametrize("staging", ["direct", "lds"])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_chunks_per_lane_paths(b3, dev, monkeypatch, k, staging):
    # each leaf lane folds k chunks; waves whose 64 lanes all hold k full chunks take the
    # fast input path (per-lane loads, or staged through LDS), the rest the bounded
    # per-lane loads: sizes cover both, partial waves, partial workgroups and tails
    monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", str(k))
    monkeypatch.setenv("BLAKE3_GPU_STAGING", staging)
    monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", QUAD_OFF)
    from blake3_merkle_tree_amd import workloads
    KiB = 1024
    lengths = [0, 1, 1024, 1025, 4 * KiB, 4 * KiB + 1, 255 * KiB, 256 * KiB, 256 * KiB + 1, 1024 * KiB - 7,
               1024 * KiB, 1024 * KiB + 1000, 2 * 1024 * KiB + 3 * KiB + 5, 3 * 1024 * KiB, 5 * 1024 * KiB + 17]
    buf = workloads.random_bytes(max(lengths), 40 + k, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(41)[0].tolist())
    outs = torch.empty((len(lengths), 32), dtype=torch.uint8, device=dev)
    for i, L in enumerate(lengths):
        b3.keyed_hash(buf[:L], key, out=outs[i])
    want = oracle.hash_batch(host, [0] * len(lengths), lengths, key * len(lengths), nthreads=NTHREADS)
    assert _digests_to_bytes(outs) == want
    # batch: whole staged waves (64 KiB messages), ragged ends, tiny messages, gap bytes
    blens = [64 * KiB] * 40 + [0, 1, 1000, 5000, 63 * KiB + 5, 65 * KiB, 300 * KiB + 9, 1024 * KiB + 3] + [1] * 20
    offs, total = workloads.pack_messages(blens)
    base = torch.full((total,), 0xA5, dtype=torch.uint8, device=dev)
    data = workloads.random_bytes(total, 42, dev)
    for o, L in zip(offs, blens):
        base[o:o + L] = data[o:o + L]
    keys = workloads.key_bytes(43, len(blens))
    out = b3.keyed_hash_batch(base, offs, blens, keys.to(dev))
    want = oracle.hash_batch(_host(base), offs, blens, keys.numpy().tobytes(), nthreads=NTHREADS)
    assert _digests_to_bytes(out) == want


# (count, length, stride): equal lengths at evenly spaced offsets take the table-free path
UNIFORM_CASES = [
    (1000, 0, 16),
    (513, 1, 16),
    (300, 1024, 1024),  # one full chunk per message: the chunk carries ROOT
    (100, 2048, 2048),
    (200, 4096, 4096),  # at four chunks per lane: one node per message, ROOT on its last parent
    (300, 3 * 1024 + 5, 4096),
    (129, 64 * 1024, 64 * 1024 + 32),
    (77, 200 * 1024 + 1, 256 * 1024),
    (50, 5000, 0),  # every message is the same bytes; the keys differ
    (9, 1024 * 1024 + 1000, 1024 * 1024 + 1024),
    (3, 4 * 1024 * 1024, 4 * 1024 * 1024),
    (40, 64 * 1024 + 1, 65 * 1024),  # 65 chunks: just past one quad-leaf workgroup
    (2, 65537 * 1024 + 3, 65537 * 1024 + 16),  # at one chunk per lane: two level passes
    (3, 600 * 256 * 1024 + 77, 600 * 256 * 1024 + 80),  # 600 leaf CVs a message at one chunk per lane
]


@pytest.mark.parametrize("staging", ["direct", "lds"])
@pytest.mark.parametrize("k", [None, 1, 4, "quad"])
def test_uniform_batches(b3, dev, monkeypatch, k, staging):
    # k: chunks per lane of the lane-per-chunk leaf (None: the default choice, which
    # sends small batches to the quad leaf), or "quad": the quad leaf for every batch
    # (K = 1 also fuses the level passes into the leaf launch; the others run them as
    # separate launches, the default)
    if k == "quad":
        monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", QUAD_ALL)
    elif k is not None:
        monkeypatch.setenv("BLAKE3_GPU_CHUNKS_PER_LANE", str(k))
        monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", QUAD_OFF)
        if k == 1:
            monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", "1")
    monkeypatch.setenv("BLAKE3_GPU_STAGING", staging)
    from blake3_merkle_tree_amd import workloads
    for ci, (count, L, stride) in enumerate(UNIFORM_CASES):
        offs = np.arange(count, dtype=np.uint64) * stride
        lengths = np.full(count, L, dtype=np.uint64)
        total = (count - 1) * stride + L + 16
        base = workloads.random_bytes(total, 50 + ci, dev)
        host = _host(base)
        keys = workloads.key_bytes(60 + ci, count)
        for keyed in (True, False):
            _say("uniform batch", count, "x", L, "stride", stride, "k", k, "keyed", keyed)
            out = b3.keyed_hash_batch(base, offs, lengths, keys.to(dev) if keyed else None)
            want = oracle.hash_batch(host, offs.tolist(), lengths.tolist(),
                                     keys.numpy().tobytes() if keyed else None, nthreads=NTHREADS)
            assert _digests_to_bytes(out) == want, (count, L, stride, keyed)
        # the same batch through the launch table
        monkeypatch.setenv("BLAKE3_GPU_BATCH_TABLE", "1")
        assert torch.equal(b3.keyed_hash_batch(base, offs, lengths, keys.to(dev)),
                           b3.keyed_hash_batch(base, offs, lengths, keys.to(dev)))
        assert _digests_to_bytes(b3.keyed_hash_batch(base, offs, lengths, keys.to(dev))) == \
            oracle.hash_batch(host, offs.tolist(), lengths.tolist(), keys.numpy().tobytes(), nthreads=NTHREADS)
        monkeypatch.delenv("BLAKE3_GPU_BATCH_TABLE")


def test_copies_run_on_the_calls_stream(b3, dev):
    # a misaligned input view and a misaligned key array are copied by the binding; the
    # copies must run on the stream the hash runs on: with torch's current stream held busy
    # by a bounded spin kernel, a copy made there would still be pending when a hash on the
    # side stream read it
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes((1 << 20) + 64, 46, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(47)[0].tolist())
    view = buf[4:4 + (1 << 20)]
    assert view.data_ptr() % 16 == 4
    lengths = [300 * 1024, 700 * 1024 + 3]
    offs = [0, 300 * 1024]
    key_bytes = workloads.key_bytes(48, 2).to(dev)
    raw = torch.empty(64 + 4, dtype=torch.uint8, device=dev)
    keys_view = raw[4:]
    keys_view.copy_(key_bytes.view(-1))
    assert keys_view.data_ptr() % 16 == 4
    side = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)  # the current stream is busy for tens of milliseconds
    got = b3.keyed_hash(view, key, stream=side)
    got_batch = b3.keyed_hash_batch(buf, offs, lengths, keys_view, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert bytes(got.cpu().tolist()) == oracle.hash(host[4:4 + (1 << 20)].tobytes(), key)
    assert _digests_to_bytes(got_batch) == oracle.hash_batch(host, offs, lengths, key_bytes.cpu().numpy().tobytes(),
                                                             nthreads=NTHREADS)


# ---- scratch: allocation failure, prior contents, repeated runs ------------------------------

def test_forced_allocation_failure_writes_nothing(b3, dev, monkeypatch):
    # a call whose scratch cannot be had returns ENOMEM and launches nothing: its output
    # keeps its prior contents; calls that need no scratch still run
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(1 << 20, 40, dev)
    key = bytes(workloads.key_bytes(41)[0].tolist())
    out = torch.full((32,), 0x5C, dtype=torch.uint8, device=dev)
    monkeypatch.setenv("BLAKE3_GPU_SCRATCH_LIMIT", "0")
    with pytest.raises(b3.Blake3GpuError) as err:
        b3.keyed_hash(buf, key, out=out)
    assert err.value.status == b3.ENOMEM
    offs, lengths = [0, 300 * 1024], [300 * 1024, 700 * 1024]
    outs = torch.full((2, 32), 0x5C, dtype=torch.uint8, device=dev)
    with pytest.raises(b3.Blake3GpuError) as err:
        b3.keyed_hash_batch(buf, offs, lengths, None, out=outs)
    assert err.value.status == b3.ENOMEM
    torch.cuda.synchronize()
    assert out.eq(0x5C).all() and outs.eq(0x5C).all()
    small = b3.keyed_hash(buf[:3000], key)  # three chunks: one leaf workgroup, no scratch
    host = _host(buf)
    assert bytes(small.cpu().tolist()) == oracle.hash(host[:3000].tobytes(), key)
    monkeypatch.delenv("BLAKE3_GPU_SCRATCH_LIMIT")
    b3.keyed_hash(buf, key, out=out)
    assert bytes(out.cpu().tolist()) == oracle.hash(host.tobytes(), key)


@pytest.mark.parametrize("fill", ["0x00", "0xA5", "0xFF"])
def test_results_do_not_depend_on_scratch_contents(b3, dev, monkeypatch, fill):
    # scratch filled with a known byte before every call's kernels: the level passes, the
    # fused level tickets, split message ends and the XOF root inputs read only what the
    # call wrote
    monkeypatch.setenv("BLAKE3_GPU_SCRATCH_FILL", fill)
    from blake3_merkle_tree_amd import workloads
    size = 70100 * 1024 - 100
    buf = workloads.random_bytes(size, 42, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(43)[0].tolist())
    for L in (1 << 20, 300 * 1024 + 5, size):
        for fused in ("0", "1"):
            monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", fused)
            _say("scratch fill", fill, "length", L, "fused", fused)
            assert bytes(b3.keyed_hash(buf[:L], key).cpu().tolist()) == oracle.hash(host[:L].tobytes(), key)
    lengths = [456 * 1024 + 7, 813 * 1024, 1725 * 1024 + 11, 3000, 1, 200 * 1024 + 5]
    offs, total = workloads.pack_messages(lengths)
    for fused in ("0", "1"):  # the batch's first level pass as its own launch, and fused
        monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", fused)
        out = b3.keyed_hash_batch(buf[:total], offs, lengths, None)
        assert _digests_to_bytes(out) == oracle.hash_batch(host[:total], offs, lengths, None, nthreads=NTHREADS)
    monkeypatch.setenv("BLAKE3_GPU_FUSED_LEVELS", "0")
    xof = b3.hash_xof(buf[:1 << 20], key, out_len=4096 + 17)
    assert bytes(xof.cpu().tolist()) == oracle.hash_xof(host[:1 << 20].tobytes(), key, out_len=4096 + 17)


def test_calls_on_several_streams_threads_and_behind_a_busy_stream(b3, dev):
    # the library's scratch slots are shared by calls on all streams and host threads:
    # every call must still get its own digest
    import threading
    from blake3_merkle_tree_amd import workloads
    sizes = [1 << 20, (3 << 20) + 5, 300 * 1024 + 5, 8 << 20]
    bufs = [workloads.random_bytes(n, 60 + i, dev) for i, n in enumerate(sizes)]
    key = bytes(workloads.key_bytes(64)[0].tolist())
    want = [oracle.hash(_host(b).tobytes(), key) for b in bufs]
    base, offs, lengths, keys_cpu = workloads.ragged_batch(dev)
    keys = keys_cpu.to(dev)
    want_batch = oracle.hash_batch(_host(base), offs, lengths, keys_cpu.numpy().tobytes(), nthreads=NTHREADS)
    streams = [torch.cuda.Stream(dev) for _ in range(4)]
    torch.cuda.synchronize()
    _say("four streams, round robin, no host synchronisation")
    outs = []
    for r in range(6):
        for i, st in enumerate(streams):
            outs.append((i, b3.keyed_hash(bufs[i], key, stream=st)))
        outs.append((-1, b3.keyed_hash_batch(base, offs, lengths, keys, stream=streams[r % 4])))
    torch.cuda.synchronize()
    for i, o in outs:
        if i < 0:
            assert _digests_to_bytes(o) == want_batch
        else:
            assert bytes(o.cpu().tolist()) == want[i], i
    _say("four host threads, one stream each")
    results, errors = {}, []

    def work(i):
        try:
            with torch.cuda.device(dev):
                res, batches = [], []
                for r in range(8):  # single hashes (scratch slots) and batches (slots and table buffers)
                    res.append(b3.keyed_hash(bufs[(i + r) % 4], key, stream=streams[i]))
                    if r % 2 == i % 2:
                        batches.append(b3.keyed_hash_batch(base, offs, lengths, keys, stream=streams[i]))
                streams[i].synchronize()
                results[i] = [bytes(x.cpu().tolist()) for x in res]
                if not all(_digests_to_bytes(o) == want_batch for o in batches):
                    errors.append(AssertionError(f"thread {i}: a batch digest differs"))
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(4):
        assert results[i] == [want[(i + r) % 4] for r in range(8)], i
    _say("calls queued behind a busy stream")
    st = streams[0]
    with torch.cuda.stream(st):
        torch.cuda._sleep(100_000_000)  # a bounded spin: the host runs far ahead of the device
    queued = [b3.keyed_hash(bufs[r % 4], key, stream=st) for r in range(12)]
    xof = b3.hash_xof(bufs[1], key, out_len=200, stream=st)
    # more batches than the library keeps pinned table buffers: the later ones are built
    # while the earlier tables still wait to be uploaded
    batches = [b3.keyed_hash_batch(base, offs, lengths, keys, stream=st) for _ in range(8)]
    st.synchronize()
    assert [bytes(o.cpu().tolist()) for o in queued] == [want[r % 4] for r in range(12)]
    assert bytes(xof.cpu().tolist()) == oracle.hash_xof(_host(bufs[1]).tobytes(), key, out_len=200)
    assert all(_digests_to_bytes(o) == want_batch for o in batches)


def test_repeated_runs_give_identical_digests(b3, dev):
    # determinism and race smoke test: the same calls, many times over, one result each
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(64 << 20, 44, dev)
    key = bytes(workloads.key_bytes(45)[0].tolist())
    outs = torch.empty((100, 32), dtype=torch.uint8, device=dev)
    for i in range(100):
        b3.keyed_hash(buf, key, out=outs[i])
    assert outs.eq(outs[0]).all()
    assert bytes(outs[0].cpu().tolist()) == oracle.hash(_host(buf).tobytes(), key)
    base, offs, lengths, keys_cpu = workloads.ragged_batch(dev)
    keys = keys_cpu.to(dev)
    first = b3.keyed_hash_batch(base, offs, lengths, keys)
    for _ in range(20):
        assert torch.equal(b3.keyed_hash_batch(base, offs, lengths, keys), first)


# ---- extendable output and subtree CVs ----------------------------------------------------

XOF_LENGTHS = [0, 1, 63, 64, 65, 1023, 1024, 1025, 2048, 2049, 5 * 1024 + 7, 64 * 1024, 300 * 1024 + 9,
               16384 * 1024 + 1, 20000 * 1024 + 3, 32768 * 1024 + 1]
XOF_OUT = [0, 1, 31, 32, 33, 64, 65, 200, 4096 + 17]


@pytest.mark.parametrize("keyed", [True, False])
def test_xof_matches_oracle(b3, dev, keyed):
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(max(XOF_LENGTHS), 70, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(71)[0].tolist()) if keyed else None
    for L in XOF_LENGTHS:
        want = oracle.hash_xof(host[:L].tobytes(), key, max(XOF_OUT))
        for n in XOF_OUT:
            _say("xof", L, "bytes ->", n, "keyed", keyed)
            got = bytes(b3.hash_xof(buf[:L], key, n).cpu().tolist())
            assert got == want[:n], (L, n)
    # a long output: many lanes, the last block cut short, a misaligned destination
    L = 3000
    want = oracle.hash_xof(host[:L].tobytes(), key, (1 << 20) + 5)
    assert bytes(b3.hash_xof(buf[:L], key, (1 << 20) + 5).cpu().numpy().tobytes()) == want
    dst = torch.zeros(1000 + 3, dtype=torch.uint8, device=dev)
    b3.hash_xof(buf[:L], key, 1000, out=dst[3:])
    assert bytes(dst[3:].cpu().numpy().tobytes()) == want[:1000]
    assert dst[:3].sum().item() == 0


@pytest.mark.parametrize("keyed", [True, False])
def test_xof_from_an_offset_matches_oracle(b3, dev, keyed):
    # reads that start mid-block, span several launches' worth of lanes, end mid-block, and
    # sit at and across multiples of 2^32 blocks (the counter's high word changes there,
    # and no launch may cross it); a misaligned destination with untouched bytes around it
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(70 * 1024 + 9, 74, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(75)[0].tolist()) if keyed else None
    wrap = 64 << 32
    cases = [(L, off, n) for L in (0, 100, 1024, 70 * 1024 + 9)
             for off, n in ((0, 64), (1, 63), (63, 2), (64, 64), (100, 1000), (5, 64 * 300 + 7),
                            (wrap - 64, 128), (wrap - 21, 50), (wrap, 64), (wrap - 64 * 700 - 3, 64 * 1400 + 9),
                            (3 * wrap + 17, 300), ((1 << 62) + 1, 200))]
    for L, off, n in cases:
        _say("xof at", off, "length", n, "input", L, "keyed", keyed)
        got = bytes(b3.hash_xof(buf[:L], key, n, offset=off).cpu().numpy().tobytes())
        assert got == oracle.hash_xof(host[:L].tobytes(), key, n, offset=off), (L, off, n)
    # the end of the 2^64-byte stream, where a block's start + 64 wraps: requests that stop
    # short of the end and requests that reach it; nothing is written past the requested
    # bytes (a guard of 64 bytes after them), and a whole wave just below the top goes
    # through the wave-wide stores
    top = 1 << 64
    for off, n in ((top - 4096, 4095), (top - 8192, 8191), (top - 65, 64), (top - 64, 63),
                   (top - 64 * 300 - 5, 64 * 300 + 4), (top - 2, 1),
                   # requests that end exactly at byte 2^64, the stream's end: its last byte
                   # is written, by the per-byte, the whole-block and the wave-wide stores
                   (top - 1, 1), (top - 5, 5), (top - 64, 64), (top - 4096, 4096), (top - 64 * 300 - 5, 64 * 300 + 5)):
        _say("xof at the top of the stream", off, "length", n, "keyed", keyed)
        guard = torch.full((n + 64,), 7, dtype=torch.uint8, device=dev)
        b3.hash_xof(buf[:5123], key, n, out=guard[:n], offset=off)
        g = guard.cpu().numpy()
        assert bytes(g[:n].tobytes()) == oracle.hash_xof(host[:5123].tobytes(), key, n, offset=off), (off, n)
        assert (g[n:] == 7).all(), (off, n)
    dst = torch.full((200 + 10,), 7, dtype=torch.uint8, device=dev)
    b3.hash_xof(buf[:1000], key, 200, out=dst[5:205], offset=wrap - 100)
    d = dst.cpu().numpy()
    assert bytes(d[5:205].tobytes()) == oracle.hash_xof(host[:1000].tobytes(), key, 200, offset=wrap - 100)
    assert (d[:5] == 7).all() and (d[205:] == 7).all()


@pytest.mark.parametrize("keyed", [True, False])
def test_subtree_cv_matches_oracle(b3, dev, keyed):
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(70000 * 1024, 72, dev)
    host = _host(buf)
    key = bytes(workloads.key_bytes(73)[0].tolist()) if keyed else None
    cases = [(0, 0), (1, 0), (1024, 5), (1025, 2), (64 * 1024, 64), (300 * 1024 + 9, 512),
             (16384 * 1024 + 1, 1 << 15), (32768 * 1024 + 1, 1 << 16), (70000 * 1024, 1 << 17),
             (5000, (1 << 40) + 8)]
    for L, base in cases:
        _say("subtree cv", L, "bytes, chunk base", base, "keyed", keyed)
        got = b3.subtree_cv(buf[:L], key, chunk_base=base).cpu().numpy().view(np.uint32).tolist()
        assert got == oracle.subtree_cv(host[:L].tobytes(), base, key), (L, base)


def _combine_share_roots(nodes, kw, mode, is_root):
    # shares are complete subtrees of 2^s chunks but the last, so over the share roots the
    # tree's left subtree is the largest power of two of shares below their count
    if len(nodes) == 1:
        return nodes[0]
    k = 1
    while 2 * k < len(nodes):
        k *= 2
    return oracle.parent_cv(kw, mode, _combine_share_roots(nodes[:k], kw, mode, False),
                            _combine_share_roots(nodes[k:], kw, mode, False), is_root=is_root)


@pytest.mark.parametrize("workload,share_chunks,cut", [("gib4", 1 << 20, None), ("fp32_8192", 1 << 15, None),
                                                       ("fp32_8192", 1 << 16, 3 * (1 << 26) - 5)])
def test_share_roots_combine_to_the_digest(b3, dev, workload, share_chunks, cut):
    # the input cut into shares of 2^s chunks, each share's root from subtree_cv with its
    # chunk base (what one GPU of several would compute), the share roots joined by parent
    # compressions on the host: the digest of the whole input (gib4: 5 shares, the last one
    # the 1000-byte tail chunk; fp32_8192: 8 shares, and 3 with a partial last share)
    import struct
    from blake3_merkle_tree_amd import workloads
    t, key = workloads.single(workload, dev)
    t = t.reshape(-1).view(torch.uint8)
    if cut is not None:
        t = t[:cut]
    key = bytes(key.tolist())
    n = t.numel()
    share_bytes = share_chunks * 1024
    p = (n + share_bytes - 1) // share_bytes
    _say("share roots", workload, n, "bytes in", p, "shares of", share_chunks, "chunks")
    roots = [b3.subtree_cv(t[g * share_bytes:min(n, (g + 1) * share_bytes)], key, chunk_base=g * share_chunks)
             .cpu().numpy().view(np.uint32).tolist() for g in range(p)]
    kw = list(struct.unpack("<8I", key))
    digest = struct.pack("<8I", *_combine_share_roots(roots, kw, oracle.KEYED_HASH, True))
    assert digest == bytes(b3.keyed_hash(t, key).cpu().tolist())
    host = _host(t)
    del t
    torch.cuda.empty_cache()
    assert digest == oracle.hash_mt(host, key, NTHREADS)


def test_graph_capture_replays_match_eager(b3, dev):
    # One graph holding a keyed hash (130 MiB + 7 B: a leaf at one chunk per lane and two level
    # passes; from 64 to 128 MiB a single message runs two chunks per lane and one pass), an XOF read
    # across a multiple of 2^32 blocks, a subtree CV with a chunk base above 2^32 and a
    # uniform batch (no task table). Replayed four times, with the outputs cleared, eager
    # hashing and synchronisations between replays: every replay gives the eager results.
    # The replay reads the inputs as they are then: a changed byte changes its digest.
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(130 * 1024 * 1024 + 7, 81, dev)
    key = bytes(workloads.key_bytes(82)[0].tolist())
    bkeys = workloads.key_bytes(83, 64).to(dev)
    boffs, blens = [4096 * i for i in range(64)], [3000] * 64
    outs = {"hash": torch.empty(32, dtype=torch.uint8, device=dev),
            "xof": torch.empty(200, dtype=torch.uint8, device=dev),
            "subtree": torch.empty(32, dtype=torch.uint8, device=dev),
            "batch": torch.empty((64, 32), dtype=torch.uint8, device=dev)}

    def run():
        b3.keyed_hash(buf, key, out=outs["hash"])
        b3.hash_xof(buf[:5000], key, 200, out=outs["xof"], offset=(64 << 32) - 100)
        b3.subtree_cv(buf[:1 << 20], key, chunk_base=1 << 33, out=outs["subtree"])
        b3.keyed_hash_batch(buf, boffs, blens, bkeys, out=outs["batch"])

    run()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in outs.items()}
    assert bytes(want["hash"].cpu().tolist()) == oracle.hash(_host(buf).tobytes(), key)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # a first run on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("capturing a single hash, an XOF, a subtree CV and a uniform batch")
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for v in outs.values():
            v.zero_()
        eager = b3.keyed_hash(buf[:12345 + rep], key)  # the library's eager path in between
        torch.cuda.synchronize()
        _say("replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], want[k]), (rep, k)
        assert bytes(eager.cpu().tolist()) == oracle.hash(_host(buf[:12345 + rep]).tobytes(), key)
    buf[130 * 1024 * 1024] ^= 0x5A
    changed = b3.keyed_hash(buf, key)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert not torch.equal(changed, want["hash"])
    assert torch.equal(outs["hash"], changed)
    del g


def test_table_batch_under_capture_is_refused(b3, dev):
    # a batch that needs a task table reads it from reused host memory: under capture the
    # call returns EINVAL and records nothing (the capture itself stays valid)
    from blake3_merkle_tree_amd import workloads
    buf = workloads.random_bytes(1 << 20, 84, dev)
    keys = workloads.key_bytes(85, 2).to(dev)
    out = torch.zeros((2, 32), dtype=torch.uint8, device=dev)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.capture_begin()
        try:
            out.fill_(7)
            with pytest.raises(b3.Blake3GpuError) as err:
                b3.keyed_hash_batch(buf, [0, 4096], [3000, 100], keys, out=out)
        finally:
            g.capture_end()
    assert err.value.status == b3.EINVAL
    g.replay()
    torch.cuda.synchronize()
    assert (out == 7).all()
    # the same batch outside capture is hashed as usual
    b3.keyed_hash_batch(buf, [0, 4096], [3000, 100], keys, out=out)
    host = _host(buf)
    assert _digests_to_bytes(out) == oracle.hash_batch(host, [0, 4096], [3000, 100], keys.cpu().numpy().tobytes())
