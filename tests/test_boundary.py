"""The C-ABI boundary without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments with the documented status codes before it
makes any HIP call (so these run on a machine with no device)."""
import ctypes
import glob
import os
import re

import pytest
import torch

import blake3_merkle_tree_amd as b3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(blake3_gpu_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"blake3_gpu_hash", "blake3_gpu_keyed_hash", "blake3_gpu_keyed_hash_batch",
            "blake3_gpu_strerror"} <= set(names)
    lib = ctypes.CDLL(b3.library_path())
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in include/ but not exported"


def _lib():
    lib = ctypes.CDLL(b3.library_path())
    vp, u64 = ctypes.c_void_p, ctypes.c_uint64
    lib.blake3_gpu_hash.argtypes = [vp, u64, vp, vp]
    lib.blake3_gpu_keyed_hash.argtypes = [vp, u64, vp, vp, vp]
    lib.blake3_gpu_keyed_hash_batch.argtypes = [vp, vp, vp, vp, vp, u64, vp]
    lib.blake3_gpu_subtree_cv.argtypes = [vp, u64, u64, vp, vp, vp]
    lib.blake3_gpu_hash_xof.argtypes = [vp, u64, vp, vp, u64, vp]
    return lib


# Fake, never dereferenced addresses: every call below must return before touching them.
ALIGNED = 0x10000
MISALIGNED = 0x10004


def test_single_argument_checks():
    lib = _lib()
    key = (ctypes.c_uint32 * 8)()
    assert lib.blake3_gpu_hash(None, 5, ALIGNED, None) == b3.EINVAL
    assert lib.blake3_gpu_hash(ALIGNED, 5, None, None) == b3.EINVAL
    assert lib.blake3_gpu_hash(MISALIGNED, 5, ALIGNED, None) == b3.EALIGN
    assert lib.blake3_gpu_hash(ALIGNED, (1 << 42) + 1, ALIGNED, None) == b3.ETOOBIG
    assert lib.blake3_gpu_keyed_hash(ALIGNED, 5, None, ALIGNED, None) == b3.EINVAL
    assert lib.blake3_gpu_keyed_hash(MISALIGNED, 5, ctypes.addressof(key), ALIGNED, None) == b3.EALIGN
    assert lib.blake3_gpu_keyed_hash(ALIGNED, 1 << 43, ctypes.addressof(key), ALIGNED, None) == b3.ETOOBIG


def test_subtree_and_xof_argument_checks():
    lib = _lib()
    assert lib.blake3_gpu_subtree_cv(ALIGNED, 5, 0, None, None, None) == b3.EINVAL
    assert lib.blake3_gpu_subtree_cv(None, 5, 0, None, ALIGNED, None) == b3.EINVAL
    assert lib.blake3_gpu_subtree_cv(MISALIGNED, 5, 0, None, ALIGNED, None) == b3.EALIGN
    assert lib.blake3_gpu_subtree_cv(ALIGNED, (1 << 42) + 1, 0, None, ALIGNED, None) == b3.ETOOBIG
    assert lib.blake3_gpu_subtree_cv(ALIGNED, 2048, (1 << 64) - 1, None, ALIGNED, None) == b3.EINVAL
    assert lib.blake3_gpu_hash_xof(ALIGNED, 5, None, None, 10, None) == b3.EINVAL
    assert lib.blake3_gpu_hash_xof(None, 5, None, ALIGNED, 10, None) == b3.EINVAL
    assert lib.blake3_gpu_hash_xof(MISALIGNED, 5, None, ALIGNED, 10, None) == b3.EALIGN
    assert lib.blake3_gpu_hash_xof(ALIGNED, 5, None, ALIGNED, (1 << 42) + 1, None) == b3.ETOOBIG
    assert lib.blake3_gpu_hash_xof(ALIGNED, 5, None, None, 0, None) == b3.OK  # nothing to write
    lib.blake3_gpu_hash_xof_at.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                           ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    assert lib.blake3_gpu_hash_xof_at(ALIGNED, 5, None, (1 << 64) - 10, ALIGNED, 20, None) == b3.EINVAL  # wraps
    assert lib.blake3_gpu_hash_xof_at(ALIGNED, 5, None, 7, None, 10, None) == b3.EINVAL
    assert lib.blake3_gpu_hash_xof_at(MISALIGNED, 5, None, 7, ALIGNED, 10, None) == b3.EALIGN
    assert lib.blake3_gpu_hash_xof_at(ALIGNED, 5, None, 7, ALIGNED, (1 << 42) + 1, None) == b3.ETOOBIG
    assert lib.blake3_gpu_hash_xof_at(ALIGNED, 5, None, (1 << 64) - 1, None, 0, None) == b3.OK
    # a request may end at byte 2^64 (the stream's last byte is 2^64 - 1), not one past it
    assert lib.blake3_gpu_hash_xof_at(ALIGNED, 5, None, (1 << 64) - 10, ALIGNED, 11, None) == b3.EINVAL
    assert lib.blake3_gpu_hash_xof_at(ALIGNED, 5, None, (1 << 64) - 1, ALIGNED, 2, None) == b3.EINVAL
    for off, n in (((1 << 64) - 10, 10), ((1 << 64) - 1, 1)):
        assert lib.blake3_gpu_hash_xof_at(MISALIGNED, 5, None, off, ALIGNED, n, None) == b3.EALIGN  # range ok


def test_group_cvs_argument_checks_and_leaf_group_size(monkeypatch):
    lib = _lib()
    lib.blake3_gpu_group_cvs.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                         ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.blake3_gpu_leaf_group_chunks.argtypes = [ctypes.c_uint64]
    lib.blake3_gpu_leaf_group_chunks.restype = ctypes.c_uint32
    for g in (0, 32, 128, 2048):  # only 64 (quad leaf), 256, 512 and 1024 are workgroup sizes
        assert lib.blake3_gpu_group_cvs(ALIGNED, 5000, 0, None, g, ALIGNED, None) == b3.EINVAL
    for g in (64, 256, 512, 1024):
        assert lib.blake3_gpu_group_cvs(ALIGNED, 0, 0, None, g, ALIGNED, None) == b3.EINVAL
        assert lib.blake3_gpu_group_cvs(None, 5000, 0, None, g, ALIGNED, None) == b3.EINVAL
        assert lib.blake3_gpu_group_cvs(ALIGNED, 5000, 0, None, g, None, None) == b3.EINVAL
        assert lib.blake3_gpu_group_cvs(MISALIGNED, 5000, 0, None, g, ALIGNED, None) == b3.EALIGN
    # what the hash entry points use: the quad leaf up to 32768 chunks, then 256 * K with the K
    # that leaves the busiest of the 256 CUs the fewest chunks per lane (the largest among
    # equals): 64 MiB is one K = 1 workgroup per CU, 192 MiB is 3 K = 1 rounds against 4 chunks
    # per lane at K = 2 or 4, 256 MiB one K = 4 round, 320 MiB 5 K = 1 rounds, 384 MiB 6 at
    # K = 2; K = 4 from 2 GiB. Up to 2^15 chunks above 2^16, 2^17 and 2^18 chunks (64 MiB + 1 B,
    # 128 MiB + 1 B, 256 MiB + 32 MiB) the power of two is one round at K = 1, 2 and 4 and the
    # rest runs on quads
    monkeypatch.delenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", raising=False)
    monkeypatch.delenv("BLAKE3_GPU_CHUNKS_PER_LANE", raising=False)
    assert [lib.blake3_gpu_leaf_group_chunks(n) for n in
            (0, 1 << 20, 32768 * 1024, 32768 * 1024 + 1, 64 << 20, (64 << 20) + 1, 128 << 20, (128 << 20) + 1,
             192 << 20, 256 << 20, (256 << 20) + (32 << 20), (256 << 20) + (32 << 20) + 1, 320 << 20, 384 << 20,
             2 << 30, (4 << 30) + 1000)] == \
        [64, 64, 64, 256, 256, 256, 512, 512, 256, 1024, 1024, 256, 256, 512, 1024, 1024]
    monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", "0")
    assert lib.blake3_gpu_leaf_group_chunks(1 << 20) == 256
    assert b3.leaf_group_chunks(1 << 20) == 256


def test_batch_argument_checks():
    lib = _lib()
    offs = (ctypes.c_uint64 * 2)(0, 32)
    lens = (ctypes.c_uint64 * 2)(10, 10)
    o, ln = ctypes.addressof(offs), ctypes.addressof(lens)
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, o, ln, None, ALIGNED, 0, None) == b3.OK  # n == 0
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, None, ln, None, ALIGNED, 2, None) == b3.EINVAL
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, o, None, None, ALIGNED, 2, None) == b3.EINVAL
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, o, ln, None, None, 2, None) == b3.EINVAL
    assert lib.blake3_gpu_keyed_hash_batch(MISALIGNED, o, ln, None, ALIGNED, 2, None) == b3.EALIGN
    assert lib.blake3_gpu_keyed_hash_batch(None, o, ln, None, ALIGNED, 2, None) == b3.EINVAL
    bad_offs = (ctypes.c_uint64 * 2)(0, 40)
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, ctypes.addressof(bad_offs), ln, None, ALIGNED, 2,
                                           None) == b3.EALIGN
    big = (ctypes.c_uint64 * 2)(10, (1 << 42) + 1)
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, o, ctypes.addressof(big), None, ALIGNED, 2,
                                           None) == b3.ETOOBIG
    # the key array is read with 16-byte loads: it must be 16-byte aligned
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, o, ln, ALIGNED + 4, ALIGNED, 2, None) == b3.EALIGN
    wrap_offs = (ctypes.c_uint64 * 2)(0, (1 << 64) - 16)
    wrap_lens = (ctypes.c_uint64 * 2)(10, 32)  # second message would wrap past 2^64
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, ctypes.addressof(wrap_offs), ctypes.addressof(wrap_lens),
                                           None, ALIGNED, 2, None) == b3.EINVAL


def test_forced_scratch_failure_returns_enomem_before_any_hip_call(monkeypatch):
    # BLAKE3_GPU_SCRATCH_LIMIT caps a call's scratch request: every call that needs
    # scratch fails with ENOMEM before any allocation or launch (no device here, so either
    # would fail with EHIP instead; the batch's graph-capture query, which enqueues
    # nothing, reads a failed query as no capture), launching nothing
    lib = _lib()
    monkeypatch.setenv("BLAKE3_GPU_SCRATCH_LIMIT", "0")
    key = (ctypes.c_uint32 * 8)()
    assert lib.blake3_gpu_hash(ALIGNED, 1 << 20, ALIGNED, None) == b3.ENOMEM  # leaf CVs + a level pass
    assert lib.blake3_gpu_keyed_hash(ALIGNED, (4 << 30) + 1000, ctypes.addressof(key), ALIGNED, None) == b3.ENOMEM
    offs = (ctypes.c_uint64 * 3)(0, 1 << 20, 3 << 20)
    lens = (ctypes.c_uint64 * 3)(300 * 1024, 2 << 20, 5)  # not uniform: the task table path
    assert lib.blake3_gpu_keyed_hash_batch(ALIGNED, ctypes.addressof(offs), ctypes.addressof(lens), None, ALIGNED,
                                           3, None) == b3.ENOMEM
    assert lib.blake3_gpu_hash_xof(ALIGNED, 1 << 20, None, ALIGNED, 64, None) == b3.ENOMEM
    assert lib.blake3_gpu_subtree_cv(ALIGNED, 1 << 20, 0, None, ALIGNED, None) == b3.ENOMEM
    monkeypatch.setenv("BLAKE3_GPU_SCRATCH_LIMIT", str(1 << 40))  # a limit no call reaches: no effect
    monkeypatch.setenv("BLAKE3_GPU_SCRATCH_LIMIT", "")  # unset or empty: no limit
    assert lib.blake3_gpu_hash(MISALIGNED, 1 << 20, ALIGNED, None) == b3.EALIGN  # checks come first


def test_noalloc_refuses_inputs_beyond_its_fixed_scratch_before_any_hip_call():
    # the fixed array (1 MiB) holds the level CVs of at most 32,640 leaf workgroups of 1024
    # chunks: one byte more is refused before any HIP call (the pointers are never
    # dereferenced); at the limit the call goes on to the device (no device here: EHIP)
    lib = b3._load()
    fake = ctypes.c_void_p(1 << 20)
    key = (ctypes.c_uint32 * 8)()
    limit = 32640 * 1024 * 1024
    assert lib.blake3_gpu_keyed_hash_noalloc(fake, limit + 1, key, fake, None) == b3.ESCRATCH
    assert lib.blake3_gpu_keyed_hash_noalloc(fake, limit + 1, None, fake, None) == b3.ESCRATCH
    assert lib.blake3_gpu_keyed_hash_noalloc(fake, 1 << 42, key, fake, None) == b3.ESCRATCH
    assert lib.blake3_gpu_keyed_hash_noalloc(fake, (1 << 42) + 1, key, fake, None) == b3.ETOOBIG
    if not torch.cuda.is_available():
        assert lib.blake3_gpu_keyed_hash_noalloc(fake, limit, key, fake, None) == b3.EHIP
    assert lib.blake3_gpu_keyed_hash_noalloc(None, 5, key, fake, None) == b3.EINVAL
    assert lib.blake3_gpu_keyed_hash_noalloc(fake, 5, key, None, None) == b3.EINVAL
    assert lib.blake3_gpu_keyed_hash_noalloc(ctypes.c_void_p(MISALIGNED), 5, key, fake, None) == b3.EALIGN


def test_environment_hooks_are_read_at_load_and_on_reload():
    # no call reads the environment: a change takes effect only when the library is asked
    # to read it again (plain os.environ here, not the test suite's reloading monkeypatch)
    lib = b3._load()
    name = "BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS"
    saved = os.environ.pop(name, None)
    lib.blake3_gpu_debug_reload_env()
    try:
        assert lib.blake3_gpu_leaf_group_chunks(1 << 20) == 64
        os.environ[name] = "0"
        assert lib.blake3_gpu_leaf_group_chunks(1 << 20) == 64  # still what was read before
        assert lib.blake3_gpu_debug_reload_env() == b3.OK
        assert lib.blake3_gpu_leaf_group_chunks(1 << 20) == 256
    finally:
        os.environ.pop(name, None)
        if saved is not None:
            os.environ[name] = saved
        lib.blake3_gpu_debug_reload_env()


def test_strerror_and_version():
    for code in (b3.OK, b3.EINVAL, b3.EALIGN, b3.ENOMEM, b3.EHIP, b3.ETOOBIG, b3.ESCRATCH):
        assert b3.strerror(code) and b3.strerror(code) != "unknown status"
    assert b3.strerror(12345) == "unknown status"
    assert b3.version() >= 10000


def test_python_binding_range_checks_64_bit_arguments():
    # ctypes reduces Python ints mod 2^64 without complaint: the binding refuses values a
    # uint64 cannot hold, before it looks at the tensor
    t = torch.zeros(16, dtype=torch.uint8)
    for call in (lambda: b3._u64(1 << 64, "x"), lambda: b3._u64(-1, "x")):
        with pytest.raises(ValueError):
            call()
    assert b3._u64((1 << 64) - 1, "x") == (1 << 64) - 1
    with pytest.raises(ValueError, match="2\\^64"):
        b3.hash_xof(t, None, 32, offset=(1 << 64) + 5)
    with pytest.raises(ValueError, match="2\\^64"):
        b3.hash_xof(t, None, 11, offset=(1 << 64) - 10)
    with pytest.raises(ValueError, match="2\\^64"):
        b3.subtree_cv(t, None, chunk_base=1 << 64)
    with pytest.raises(ValueError, match="2\\^64"):
        b3.group_cvs(t, None, chunk_base=(1 << 64) + 7)
    with pytest.raises(ValueError, match="HIP device"):  # in range: on to the tensor check
        b3.hash_xof(t, None, 10, offset=(1 << 64) - 10)


def test_python_binding_rejects_host_tensors_and_bad_keys():
    with pytest.raises(ValueError):
        b3.hash(torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        b3.keyed_hash(torch.zeros(16, dtype=torch.uint8), bytes(32))
    with pytest.raises(ValueError):
        b3._key_words(b"short")
    with pytest.raises(ValueError):
        b3.keyed_hash_batch(torch.zeros(16, dtype=torch.uint8), [0], [16])


def test_missing_library_raises_and_nothing_falls_back(monkeypatch, tmp_path):
    # the binding has no CPU path: with its library absent, every call that would reach the
    # library raises ImportError rather than computing anything another way
    monkeypatch.setattr(b3, "_LIB_PATH", str(tmp_path / "libblake3_gpu.so"))
    monkeypatch.setattr(b3, "_lib", None)
    calls = [lambda: b3.version(), lambda: b3.strerror(0), lambda: b3.leaf_group_chunks(1 << 20),
             lambda: b3.debug_plan_batch([1024, 5])]
    for call in calls:
        with pytest.raises(ImportError, match="is not built"):
            call()


def test_more_leaf_workgroups_than_one_grid_is_too_big(monkeypatch):
    # a quad leaf (64 chunks per workgroup) forced onto 2^42 bytes would need 2^26 workgroups
    # for one message, more than one launch holds: the call refuses before any HIP call
    # (the pointers are never dereferenced)
    monkeypatch.setenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS", str(1 << 40))
    lib = b3._load()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.blake3_gpu_hash(fake, 1 << 42, fake, None) == b3.ETOOBIG
    monkeypatch.delenv("BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS")


def test_group_cvs_refuses_more_groups_than_one_launch():
    # 2^42 bytes in groups of 64 chunks is 2^26 workgroups, in groups of 256 chunks 2^24:
    # both more than one launch's 2^32 - 1 work-items (256 per workgroup); 512 chunks fit.
    # The call refuses before any HIP call (the pointers are never dereferenced).
    lib = b3._load()
    fake = ctypes.c_void_p(1 << 20)
    key = (ctypes.c_uint32 * 8)()
    for group in (64, 256):
        assert lib.blake3_gpu_group_cvs(fake, 1 << 42, 0, key, group, fake, None) == b3.ETOOBIG, group
    assert lib.blake3_gpu_group_cvs(fake, (1 << 42) + 1, 0, key, 1024, fake, None) == b3.ETOOBIG
