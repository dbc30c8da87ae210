"""ctypes binding of the plain CPU BLAKE3 oracle (oracle/blake3_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by the
CPU-baseline leg of bench.py. The product package never imports it.

Byte inputs may be ``bytes``, ``bytearray``, ``memoryview`` or a C-contiguous numpy
uint8 array; keys are 32 bytes (or None for default, unkeyed mode); digests are
returned as 32-byte ``bytes``.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)

CHUNK_LEN = 1024
BLOCK_LEN = 64
# Flag bits of the BLAKE3 specification (restated for callers of compress()).
CHUNK_START, CHUNK_END, PARENT, ROOT, KEYED_HASH = 1, 2, 4, 8, 16


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(LIB)
    lib.b3o_round.argtypes = [_u32p, _u32p]
    lib.b3o_iv.argtypes = [_u32p]
    lib.b3o_compress.argtypes = [_u32p, _u32p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, _u32p]
    lib.b3o_chunk_cv.argtypes = [_u32p, ctypes.c_uint32, _u8p, ctypes.c_size_t, ctypes.c_uint64,
                                 ctypes.c_int, _u32p]
    lib.b3o_parent_cv.argtypes = [_u32p, ctypes.c_uint32, _u32p, _u32p, ctypes.c_int, _u32p]
    lib.b3o_left_subtree_chunks.argtypes = [ctypes.c_uint64]
    lib.b3o_left_subtree_chunks.restype = ctypes.c_uint64
    lib.b3o_hash_recursive.argtypes = [_u8p, ctypes.c_uint64, _u8p, _u8p]
    lib.b3o_subtree_cv.argtypes = [_u8p, ctypes.c_uint64, ctypes.c_uint64, _u8p, _u32p]
    lib.b3o_hash_xof.argtypes = [_u8p, ctypes.c_uint64, _u8p, _u8p, ctypes.c_uint64]
    lib.b3o_hash_xof_at.argtypes = [_u8p, ctypes.c_uint64, _u8p, ctypes.c_uint64, _u8p, ctypes.c_uint64]
    lib.b3o_hasher_new.argtypes = [_u8p]
    lib.b3o_hasher_new.restype = ctypes.c_void_p
    lib.b3o_hasher_free.argtypes = [ctypes.c_void_p]
    lib.b3o_hasher_update.argtypes = [ctypes.c_void_p, _u8p, ctypes.c_uint64]
    lib.b3o_hasher_finalize.argtypes = [ctypes.c_void_p, _u8p]
    lib.b3o_hash.argtypes = [_u8p, ctypes.c_uint64, _u8p]
    lib.b3o_keyed_hash.argtypes = [_u8p, ctypes.c_uint64, _u8p, _u8p]
    lib.b3o_hash_mt.argtypes = [_u8p, ctypes.c_uint64, _u8p, _u8p, ctypes.c_int]
    lib.b3o_hash_mt.restype = ctypes.c_int
    lib.b3o_hash_batch.argtypes = [_u8p, _u64p, _u64p, ctypes.c_uint64, _u8p, _u8p, ctypes.c_int]
    lib.b3o_hash_batch.restype = ctypes.c_int
    _lib = lib
    return lib


def _as_u8(data):
    """Return (numpy uint8 view, ctypes pointer) without copying when possible."""
    if isinstance(data, np.ndarray):
        arr = np.ascontiguousarray(data).view(np.uint8).reshape(-1)
    else:
        arr = np.frombuffer(memoryview(data).cast("B"), dtype=np.uint8)
    if arr.size == 0:
        arr = np.zeros(1, dtype=np.uint8)[:0]
    return arr, arr.ctypes.data_as(_u8p)


def _key(key):
    if key is None:
        return None, None
    k = np.frombuffer(bytes(key), dtype=np.uint8)
    if k.size != 32:
        raise ValueError("BLAKE3 keys are 32 bytes")
    return k, k.ctypes.data_as(_u8p)


def _words(seq, n):
    arr = (ctypes.c_uint32 * n)(*[int(x) & 0xFFFFFFFF for x in seq])
    return arr


def iv():
    out = (ctypes.c_uint32 * 8)()
    _load().b3o_iv(out)
    return list(out)


def round_fn(v, m):
    """One BLAKE3/BLAKE2s-layout round on a 16-word state with 16 message words."""
    vv = _words(v, 16)
    _load().b3o_round(vv, _words(m, 16))
    return list(vv)


def compress(cv, block_words, counter, block_len, flags):
    """Full 16-word output of the compression function."""
    out = (ctypes.c_uint32 * 16)()
    _load().b3o_compress(_words(cv, 8), _words(block_words, 16), counter, block_len, flags, out)
    return list(out)


def chunk_cv(key_words, mode, chunk, chunk_index, is_root=False):
    arr, ptr = _as_u8(chunk)
    out = (ctypes.c_uint32 * 8)()
    _load().b3o_chunk_cv(_words(key_words, 8), mode, ptr, arr.size, chunk_index, int(is_root), out)
    return list(out)


def parent_cv(key_words, mode, left, right, is_root=False):
    out = (ctypes.c_uint32 * 8)()
    _load().b3o_parent_cv(_words(key_words, 8), mode, _words(left, 8), _words(right, 8), int(is_root), out)
    return list(out)


def left_subtree_chunks(n):
    return int(_load().b3o_left_subtree_chunks(n))


def hash_recursive(data, key=None):
    arr, ptr = _as_u8(data)
    _, kp = _key(key)
    out = (ctypes.c_uint8 * 32)()
    _load().b3o_hash_recursive(ptr, arr.size, kp, out)
    return bytes(out)


def subtree_cv(data, chunk_base=0, key=None):
    """8-word CV (no ROOT) of the subtree over all chunks of `data`, first counter chunk_base."""
    arr, ptr = _as_u8(data)
    _k, kp = _key(key)
    out = (ctypes.c_uint32 * 8)()
    _load().b3o_subtree_cv(ptr, arr.size, chunk_base, kp, out)
    return list(out)


def hash_xof(data, key=None, out_len=32, offset=0):
    """Extended output: bytes [offset, offset + out_len) of the root node's output stream
    (blocks of 64 bytes, counter 0, 1, ...); the first 32 bytes are the hash."""
    arr, ptr = _as_u8(data)
    _k, kp = _key(key)
    out = (ctypes.c_uint8 * max(int(out_len), 1))()
    _load().b3o_hash_xof_at(ptr, arr.size, kp, int(offset), out, int(out_len))
    return bytes(out)[:int(out_len)]


def hash(data, key=None):  # noqa: A001 - mirrors the spec's name
    """One-shot hash through the incremental (stack-merge) form."""
    arr, ptr = _as_u8(data)
    out = (ctypes.c_uint8 * 32)()
    if key is None:
        _load().b3o_hash(ptr, arr.size, out)
    else:
        k, kp = _key(key)
        _load().b3o_keyed_hash(ptr, arr.size, kp, out)
    return bytes(out)


def hash_mt(data, key=None, nthreads=None):
    arr, ptr = _as_u8(data)
    k, kp = _key(key)
    out = (ctypes.c_uint8 * 32)()
    nthreads = nthreads or os.cpu_count() or 1
    if _load().b3o_hash_mt(ptr, arr.size, kp, out, int(nthreads)) != 0:
        raise MemoryError("oracle multi-threaded hash failed")
    return bytes(out)


def hash_batch(base, offsets, lengths, keys=None, nthreads=None):
    """Hash n messages base[offsets[i]:offsets[i]+lengths[i]]; keys: n*32 bytes or None."""
    arr, ptr = _as_u8(base)
    offs = np.ascontiguousarray(offsets, dtype=np.uint64)
    lens = np.ascontiguousarray(lengths, dtype=np.uint64)
    n = offs.size
    if lens.size != n:
        raise ValueError("offsets and lengths differ in size")
    if n and int((offs + lens).max()) > arr.size:
        raise ValueError("a message runs past the end of the buffer")
    kp = None
    if keys is not None:
        karr = np.ascontiguousarray(np.frombuffer(bytes(keys), dtype=np.uint8))
        if karr.size != 32 * n:
            raise ValueError("keys must hold 32 bytes per message")
        kp = karr.ctypes.data_as(_u8p)
    out = np.zeros(32 * max(n, 1), dtype=np.uint8)
    nthreads = nthreads or os.cpu_count() or 1
    _load().b3o_hash_batch(ptr, offs.ctypes.data_as(_u64p), lens.ctypes.data_as(_u64p), n, kp,
                           out.ctypes.data_as(_u8p), int(nthreads))
    return [bytes(out[32 * i: 32 * i + 32]) for i in range(n)]


class Hasher:
    """Incremental hasher (stack-merge form)."""

    def __init__(self, key=None):
        self._k, kp = _key(key)
        self._h = _load().b3o_hasher_new(kp)
        if not self._h:
            raise MemoryError

    def update(self, data):
        arr, ptr = _as_u8(data)
        _load().b3o_hasher_update(self._h, ptr, arr.size)
        return self

    def digest(self):
        out = (ctypes.c_uint8 * 32)()
        _load().b3o_hasher_finalize(self._h, out)
        return bytes(out)

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.b3o_hasher_free(self._h)
            self._h = None
