"""BLAKE3 Merkle-tree hashing of GPU-resident buffers on MI355X (gfx950).

Thin ctypes binding of ``libblake3_gpu.so`` (the C ABI in ``include/blake3_gpu.h``).
PyTorch supplies device memory and streams only: every step of the hash runs in the
library's HIP kernels. The functions mirror the C entry points:

    hash(t)                              -> 32-byte digest tensor on t's device
    keyed_hash(t, key)                   -> 32-byte digest tensor (key: 32 bytes)
    keyed_hash_noalloc(t, key, out)      -> keyed_hash (or hash, key None) that allocates
                                         nothing, writing into out
    keyed_hash_batch(base, offsets, lengths, keys=None) -> (n, 32) digest tensor
    hash_xof(t, key=None, out_len=32, offset=0) -> bytes [offset, offset + out_len) of the
                                         extended output
    subtree_cv(t, key=None, chunk_base=0) -> CV (no ROOT) of the tree over t's chunks
    group_cvs(t, key=None, chunk_base=0, group_chunks=256) -> the leaf pass's group CVs
    leaf_group_chunks(nbytes)            -> chunks per leaf workgroup the hashes use

Each of the device calls also takes out= (a preallocated contiguous device tensor of the
result's size) and stream= (a torch.cuda.Stream; default: the device's current stream).
All work, including the copy the binding makes of a non-contiguous or misaligned input,
is enqueued on that stream and nothing waits for it: read a result after synchronising
the stream. A tensor is hashed as its raw bytes in memory order (a contiguous fp32 tensor
as its little-endian element bytes). There is no CPU fallback: if the library is missing
or no HIP device is present the calls raise.
"""
import contextlib
import ctypes
import functools
import os
import struct

import numpy as np
import torch

__all__ = ["hash", "keyed_hash", "keyed_hash_noalloc", "keyed_hash_batch", "hash_xof", "subtree_cv", "group_cvs", "leaf_group_chunks",
           "strerror", "version", "Blake3GpuError", "library_path", "debug_plan_batch"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libblake3_gpu.so")
_lib = None

OK, EINVAL, EALIGN, ENOMEM, EHIP, ETOOBIG, ESCRATCH = 0, -1, -2, -3, -4, -5, -6


class Blake3GpuError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python blake3_merkle_tree_amd/build.py")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, u64 = ctypes.c_void_p, ctypes.c_uint64
    lib.blake3_gpu_hash.argtypes = [vp, u64, vp, vp]
    lib.blake3_gpu_keyed_hash.argtypes = [vp, u64, ctypes.POINTER(ctypes.c_uint32), vp, vp]
    lib.blake3_gpu_keyed_hash_noalloc.argtypes = [vp, u64, ctypes.POINTER(ctypes.c_uint32), vp, vp]
    lib.blake3_gpu_keyed_hash_batch.argtypes = [vp, vp, vp, vp, vp, u64, vp]
    lib.blake3_gpu_group_cvs.argtypes = [vp, u64, u64, ctypes.POINTER(ctypes.c_uint32), ctypes.c_uint32, vp, vp]
    lib.blake3_gpu_subtree_cv.argtypes = [vp, u64, u64, ctypes.POINTER(ctypes.c_uint32), vp, vp]
    lib.blake3_gpu_hash_xof.argtypes = [vp, u64, ctypes.POINTER(ctypes.c_uint32), vp, u64, vp]
    lib.blake3_gpu_hash_xof_at.argtypes = [vp, u64, ctypes.POINTER(ctypes.c_uint32), u64, vp, u64, vp]
    lib.blake3_gpu_leaf_group_chunks.argtypes = [u64]
    lib.blake3_gpu_leaf_group_chunks.restype = ctypes.c_uint32
    lib.blake3_gpu_strerror.argtypes = [ctypes.c_int]
    lib.blake3_gpu_strerror.restype = ctypes.c_char_p
    lib.blake3_gpu_version.argtypes = []
    lib.blake3_gpu_debug_reload_env.argtypes = []
    lib.blake3_gpu_debug_reload_env.restype = ctypes.c_int
    lib.debug_plan = lib.blake3_gpu_debug_plan_batch
    lib.debug_plan.argtypes = [ctypes.POINTER(u64), u64, ctypes.POINTER(u64), u64]
    lib.debug_plan.restype = ctypes.c_int64
    for f in ("blake3_gpu_hash", "blake3_gpu_keyed_hash", "blake3_gpu_keyed_hash_noalloc",
              "blake3_gpu_keyed_hash_batch", "blake3_gpu_group_cvs",
              "blake3_gpu_subtree_cv", "blake3_gpu_hash_xof", "blake3_gpu_hash_xof_at", "blake3_gpu_version"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return _load().blake3_gpu_strerror(int(status)).decode()


def version() -> int:
    return int(_load().blake3_gpu_version())


def _check(rc, where):
    if rc != OK:
        raise Blake3GpuError(rc, where)


def _check_tensor(t, what="the tensor"):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor for {what}")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on a HIP device")


@contextlib.contextmanager
def _on(device, stream):
    """Device and stream of one call (stream None: the device's current stream); yields
    the stream's handle. The copies and outputs the binding makes are made inside it, on
    the call's stream, so that a copy is ordered before the kernels that read it and the
    allocator reuses its memory only in that stream's order. When the call runs on the
    current device's current stream there is nothing to switch."""
    if stream is None and device.index == torch.cuda.current_device():
        yield ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
        return
    with torch.cuda.device(device):
        s = stream if stream is not None else torch.cuda.current_stream(device)
        with torch.cuda.stream(s):
            yield ctypes.c_void_p(s.cuda_stream)


def _aligned(t: torch.Tensor) -> torch.Tensor:
    """The tensor's bytes as a contiguous, 16-byte-aligned device tensor (no copy if it
    already is one). Call inside _on."""
    if not t.is_contiguous():
        t = t.contiguous()
    if t.numel() and t.data_ptr() % 16 != 0:
        t = t.clone()  # fresh allocations are 256-byte aligned
    return t


def _key_words(key):
    if isinstance(key, torch.Tensor):
        key = bytes(key.detach().to("cpu", torch.uint8).contiguous().numpy().tobytes())
    key = bytes(key)
    if len(key) != 32:
        raise ValueError("BLAKE3 keys are 32 bytes")
    return _words_of_key(key)


@functools.lru_cache(maxsize=64)
def _words_of_key(key: bytes):
    # the C call reads the words during the call only, so one array can serve every call
    return (ctypes.c_uint32 * 8)(*struct.unpack("<8I", key))


def _u64_array(v, what):
    """A sequence of non-negative integers as a contiguous uint64 host array (no copy for
    a uint64 numpy array or CPU tensor)."""
    if isinstance(v, torch.Tensor):
        v = v.detach().cpu().numpy()
    if isinstance(v, np.ndarray):
        if v.dtype.kind not in "iu":
            raise TypeError(f"{what} must hold integers")
        if v.dtype.kind == "i" and v.size and int(v.min()) < 0:
            raise ValueError(f"{what} must be non-negative")
        return np.ascontiguousarray(v.reshape(-1), dtype=np.uint64)
    try:
        return np.asarray(v, dtype=np.uint64).reshape(-1)
    except OverflowError:
        raise ValueError(f"{what} must be non-negative 64-bit integers") from None


_U64_LIMIT = 1 << 64


def _u64(v, what):
    """A non-negative integer below 2^64 (ctypes would silently reduce larger ones mod 2^64)."""
    v = int(v)
    if v < 0 or v >= _U64_LIMIT:
        raise ValueError(f"{what} must be in [0, 2^64)")
    return v


def _out(out, device, n):
    if out is None:
        return torch.empty(n, dtype=torch.uint8, device=device)
    if out.device != device or out.dtype != torch.uint8 or out.numel() != n or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous uint8 tensor of {n} bytes on {device}")
    return out


def hash(t: torch.Tensor, out=None, stream=None) -> torch.Tensor:  # noqa: A001
    """Default-mode BLAKE3 of the tensor's bytes; returns a 32-byte uint8 device tensor."""
    _check_tensor(t)
    with _on(t.device, stream) as sh:
        t = _aligned(t)
        out = _out(out, t.device, 32)
        nbytes = t.numel() * t.element_size()
        rc = _load().blake3_gpu_hash(ctypes.c_void_p(t.data_ptr() if nbytes else 0), nbytes,
                                     ctypes.c_void_p(out.data_ptr()), sh)
    _check(rc, "blake3_gpu_hash")
    return out


def keyed_hash(t: torch.Tensor, key, out=None, stream=None) -> torch.Tensor:
    """Keyed-mode BLAKE3 (key: 32 bytes) of the tensor's bytes; 32-byte device tensor."""
    _check_tensor(t)
    kw = _key_words(key)
    with _on(t.device, stream) as sh:
        t = _aligned(t)
        out = _out(out, t.device, 32)
        nbytes = t.numel() * t.element_size()
        rc = _load().blake3_gpu_keyed_hash(ctypes.c_void_p(t.data_ptr() if nbytes else 0), nbytes, kw,
                                           ctypes.c_void_p(out.data_ptr()), sh)
    _check(rc, "blake3_gpu_keyed_hash")
    return out


def keyed_hash_noalloc(t: torch.Tensor, key, out: torch.Tensor, stream=None) -> torch.Tensor:
    """keyed_hash (key: 32 bytes) or hash (key None) through the entry point that allocates
    nothing: its scratch is a fixed 1 MiB device array per GPU, shared by every such call
    on that GPU, so calls that overlap on one GPU race (calls ordered on one stream do
    not). Neither the binding nor the library allocates: t must be a contiguous, 16-byte
    aligned device tensor (it is not copied) and out a contiguous 32-byte uint8 tensor on
    its device. Inputs above 31.875 GiB raise Blake3GpuError (ESCRATCH)."""
    _check_tensor(t)
    if not t.is_contiguous() or (t.numel() and t.data_ptr() % 16 != 0):
        raise ValueError("keyed_hash_noalloc copies nothing: t must be contiguous and 16-byte aligned")
    if out is None:
        raise ValueError("keyed_hash_noalloc allocates nothing: pass out (32 bytes)")
    kw = _key_words(key) if key is not None else None
    with _on(t.device, stream) as sh:
        out = _out(out, t.device, 32)
        nbytes = t.numel() * t.element_size()
        rc = _load().blake3_gpu_keyed_hash_noalloc(ctypes.c_void_p(t.data_ptr() if nbytes else 0), nbytes, kw,
                                                   ctypes.c_void_p(out.data_ptr()), sh)
    _check(rc, "blake3_gpu_keyed_hash_noalloc")
    return out


def keyed_hash_batch(base: torch.Tensor, offsets, lengths, keys=None, out=None, stream=None) -> torch.Tensor:
    """Hash messages base[offsets[i] : offsets[i] + lengths[i]] (byte offsets into the
    tensor's bytes, multiples of 16; offsets and lengths are sequences, numpy arrays or
    CPU tensors). keys: None (default mode) or a device tensor with 32 bytes per message,
    shape (n, 32) uint8 or (n, 8) int32. Returns (n, 32) uint8. Equal lengths at evenly
    spaced offsets take a faster path that needs no launch table. A base or keys tensor
    that is not 16-byte aligned is copied first (on the call's stream). Under graph
    capture only such uniform batches can be recorded: a batch that needs a launch table
    raises Blake3GpuError (EINVAL) there. Offsets or lengths given as device tensors are
    copied to the host, which waits for the device."""
    if not isinstance(base, torch.Tensor) or base.device.type != "cuda":
        raise ValueError("base must be a tensor on a HIP device")
    if not base.is_contiguous():
        raise ValueError("base must be contiguous (offsets address its bytes)")
    offs = _u64_array(offsets, "offsets")
    lens = _u64_array(lengths, "lengths")
    n = len(offs)
    if len(lens) != n:
        raise ValueError("offsets and lengths differ in size")
    nbytes = base.numel() * base.element_size()
    if n:
        ends = offs + lens  # uint64: a wrap shows as an end below its offset
        if bool((ends < offs).any()) or int(ends.max()) > nbytes:
            raise ValueError("a message runs past the end of base")
    if keys is not None:
        if not isinstance(keys, torch.Tensor) or keys.device != base.device or not keys.is_contiguous():
            raise ValueError("keys must be a contiguous tensor on base's device")
        if keys.numel() * keys.element_size() != 32 * n:
            raise ValueError("keys must hold 32 bytes per message")
    with _on(base.device, stream) as sh:
        base = _aligned(base)
        kp = ctypes.c_void_p(_aligned(keys).data_ptr() if keys is not None else 0)
        out = _out(out, base.device, 32 * n).view(n, 32) if n else torch.empty((0, 32), dtype=torch.uint8,
                                                                               device=base.device)
        rc = _load().blake3_gpu_keyed_hash_batch(ctypes.c_void_p(base.data_ptr() if nbytes else 0),
                                                 offs.ctypes.data, lens.ctypes.data,
                                                 kp, ctypes.c_void_p(out.data_ptr()), n, sh)
    _check(rc, "blake3_gpu_keyed_hash_batch")
    return out


def hash_xof(t: torch.Tensor, key=None, out_len: int = 32, out=None, stream=None, offset: int = 0) -> torch.Tensor:
    """Extendable output: bytes [offset, offset + out_len) of the root node's output stream
    for the tensor's bytes (key: 32 bytes for keyed mode, None for default mode); a uint8
    device tensor. Bytes 0..31 of the stream are the hash."""
    out_len, offset = _u64(out_len, "out_len"), _u64(offset, "offset")
    if offset + out_len > _U64_LIMIT:
        raise ValueError("the output stream is 2^64 bytes: offset + out_len must not exceed 2^64")
    _check_tensor(t)
    kw = _key_words(key) if key is not None else None
    with _on(t.device, stream) as sh:
        t = _aligned(t)
        out = _out(out, t.device, out_len)
        nbytes = t.numel() * t.element_size()
        rc = _load().blake3_gpu_hash_xof_at(ctypes.c_void_p(t.data_ptr() if nbytes else 0), nbytes, kw, offset,
                                            ctypes.c_void_p(out.data_ptr() if out_len else 0), out_len, sh)
    _check(rc, "blake3_gpu_hash_xof_at")
    return out


def subtree_cv(t: torch.Tensor, key=None, chunk_base: int = 0, out=None, stream=None) -> torch.Tensor:
    """CV (no ROOT) of the subtree over all chunks of the tensor's bytes, chunk counters
    from chunk_base: an (8,) int32 device tensor of little-endian words."""
    chunk_base = _u64(chunk_base, "chunk_base")
    _check_tensor(t)
    if out is not None and (out.device != t.device or out.numel() * out.element_size() != 32
                            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous device tensor of 32 bytes")
    kw = _key_words(key) if key is not None else None
    with _on(t.device, stream) as sh:
        t = _aligned(t)
        if out is None:
            out = torch.empty(8, dtype=torch.int32, device=t.device)
        nbytes = t.numel() * t.element_size()
        rc = _load().blake3_gpu_subtree_cv(ctypes.c_void_p(t.data_ptr() if nbytes else 0), nbytes,
                                           int(chunk_base), kw, ctypes.c_void_p(out.data_ptr()), sh)
    _check(rc, "blake3_gpu_subtree_cv")
    return out


def leaf_group_chunks(nbytes: int) -> int:
    """Chunks per leaf workgroup the hash calls use for an input of nbytes bytes."""
    return int(_load().blake3_gpu_leaf_group_chunks(int(nbytes)))


def group_cvs(t: torch.Tensor, key=None, chunk_base: int = 0, group_chunks: int = 256, out=None,
              stream=None) -> torch.Tensor:
    """CVs (no ROOT) of the aligned groups of group_chunks chunks (64: the small-input leaf
    with four lanes per chunk; 256, 512 or 1024) of the tensor's bytes, chunk counters
    starting at chunk_base: a (groups, 8) int32 device tensor of little-endian words."""
    chunk_base = _u64(chunk_base, "chunk_base")
    _check_tensor(t)
    nbytes = t.numel() * t.element_size()
    if nbytes == 0:
        raise ValueError("group_cvs needs at least one byte")
    groups = ((nbytes + 1023) // 1024 + group_chunks - 1) // group_chunks
    if out is not None and (out.device != t.device or out.numel() * out.element_size() != 32 * groups
                            or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous device tensor of {32 * groups} bytes")
    kw = _key_words(key) if key is not None else None
    with _on(t.device, stream) as sh:
        t = _aligned(t)
        if out is None:
            out = torch.empty((groups, 8), dtype=torch.int32, device=t.device)
        rc = _load().blake3_gpu_group_cvs(ctypes.c_void_p(t.data_ptr()), nbytes, int(chunk_base), kw,
                                          int(group_chunks), ctypes.c_void_p(out.data_ptr()), sh)
    _check(rc, "blake3_gpu_group_cvs")
    return out


def debug_plan_batch(lengths):
    """The batch planner's launch plan for messages of these byte lengths (no GPU work):
    a list of passes, each a dict with lanes, chunks_per_lane, in_cvs, out_cvs,
    wg_first_seg, wg_levels and segs as (msg, first, dst, lane_start, nodes, final, pair)
    tuples (pass 0: `first` is a chunk index and a node covers chunks_per_lane chunks;
    `pair`: the segment's last node is the parent of input CVs first+nodes-1 and
    first+nodes)."""
    lib = _load()
    lens = (ctypes.c_uint64 * len(lengths))(*[int(x) for x in lengths])
    need = lib.debug_plan(lens, len(lens), None, 0)
    if need < 0:
        raise Blake3GpuError(int(need), "blake3_gpu_debug_plan_batch")
    buf = (ctypes.c_uint64 * need)()
    lib.debug_plan(lens, len(lens), buf, need)
    words = list(buf)
    pos = 1
    passes = []
    for _ in range(words[0]):
        lanes, cpl, nwg, nseg, in_cvs, out_cvs = words[pos:pos + 6]
        pos += 6
        first = words[pos:pos + nwg + 1]
        pos += nwg + 1
        levels = words[pos:pos + nwg]
        pos += nwg
        segs = []
        for i in range(nseg):
            msg, f, dst, info = words[pos + 4 * i:pos + 4 * i + 4]
            segs.append((msg, f, dst, info & 0xFFF, ((info >> 12) & 0xFFF) + 1, bool(info >> 31),
                         bool((info >> 30) & 1)))
        pos += 4 * nseg
        passes.append(dict(lanes=lanes, chunks_per_lane=cpl, in_cvs=in_cvs, out_cvs=out_cvs,
                           wg_first_seg=first, wg_levels=levels, segs=segs))
    return passes
