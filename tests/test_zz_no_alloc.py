"""blake3_gpu_keyed_hash_noalloc, the entry point that allocates nothing, called through the
C ABI (ctypes on libblake3_gpu.so): its digests equal blake3_gpu_keyed_hash's (and, with a
NULL key, blake3_gpu_hash's) bit for bit on calls in a row whose inputs shrink. Every such
call on the GPU shares one fixed scratch array, so each call after the first finds there
what the previous one left; the result must not depend on it."""
import ctypes

import pytest
import torch

import blake3_merkle_tree_amd as b3
import oracle
from blake3_merkle_tree_amd import workloads

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0)


def _keyed(fn, data, key_words, stream):
    out = torch.empty(32, dtype=torch.uint8, device=data.device)
    rc = fn(_ptr(data), data.numel(), key_words, ctypes.c_void_p(out.data_ptr()), stream)
    assert rc == b3.OK, b3.strerror(rc)
    return out


def _default(lib, data, stream):
    out = torch.empty(32, dtype=torch.uint8, device=data.device)
    rc = lib.blake3_gpu_hash(_ptr(data), data.numel(), ctypes.c_void_p(out.data_ptr()), stream)
    assert rc == b3.OK, b3.strerror(rc)
    return out


def _compare(sizes, seed0, check_oracle_up_to=4 << 20):
    dev = torch.device("cuda:0")
    lib = b3._load()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for i, n in enumerate(sizes):
        print(f"no-alloc call {i}: {n} bytes", flush=True)
        data = workloads.random_bytes(n, seed0 + i, dev)
        key = bytes(workloads.key_bytes(seed0 + 100 + i)[0].tolist())
        kw = b3._key_words(key)
        got = _keyed(lib.blake3_gpu_keyed_hash_noalloc, data, kw, stream)
        got_default = _keyed(lib.blake3_gpu_keyed_hash_noalloc, data, None, stream)
        want = _keyed(lib.blake3_gpu_keyed_hash, data, kw, stream)
        want_default = _default(lib, data, stream)
        torch.cuda.synchronize()
        assert bytes(got.cpu().tolist()) == bytes(want.cpu().tolist()), n
        assert bytes(got_default.cpu().tolist()) == bytes(want_default.cpu().tolist()), n
        if n <= check_oracle_up_to:
            assert bytes(got.cpu().tolist()) == oracle.hash(data.cpu().numpy(), key), n


def test_noalloc_equals_keyed_hash_on_consecutive_shrinking_calls():
    # 128 MiB + 777 B: 513 leaf workgroups and two level passes (both CV arrays of the fixed
    # scratch); then smaller inputs: 64 MiB + 777 B (two chunks per lane, 129 leaf
    # workgroups and one level pass), the quad leaf and one level pass, a message that one
    # leaf workgroup finishes (no scratch), a short chunk, the empty input
    _compare([(128 << 20) + 777, (64 << 20) + 777, (300 << 10) + 5, 40 * 1024, 5000, 0], 700)


def test_noalloc_equals_keyed_hash_at_the_headline_size_then_smaller():
    # 4 GiB + 1000 B (4097 leaf workgroups of 1024 chunks, two level passes), then 1 MiB
    _compare([(4 << 30) + 1000, 1 << 20], 710)


def test_noalloc_binding_allocates_nothing_itself():
    dev = torch.device("cuda:0")
    data = workloads.random_bytes(3 << 20, 720, dev)
    key = bytes(workloads.key_bytes(721)[0].tolist())
    out = torch.empty(32, dtype=torch.uint8, device=dev)
    assert b3.keyed_hash_noalloc(data, key, out) is out
    want = b3.keyed_hash(data, key)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    with pytest.raises(ValueError):
        b3.keyed_hash_noalloc(data, key, None)
    with pytest.raises(ValueError):
        b3.keyed_hash_noalloc(data[1:], key, out)  # misaligned: the binding would have to copy
