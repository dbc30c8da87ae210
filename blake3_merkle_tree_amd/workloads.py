"""Seeded synthetic inputs for the hashing workloads (no hash arithmetic here).

Shared by the tests, the smoke check and the benchmark: both the GPU path and the CPU
oracle hash the bytes made here (the oracle after a device-to-host copy). Message bytes
come from torch's generator on the target device (fast for GiB inputs; the exact bytes
depend on the device kind, which does not matter because both sides read the same
buffer). Keys and message lengths come from a CPU generator, so they are identical on
every machine.

Workloads (name: what it is):
  mib1       one keyed hash of 1,048,576 uniform random bytes (1024 chunks); bytes seed 0,
             key seed 1
  ragged256  256 keyed hashes; lengths 0, 1, 63, 64, 65, 1023, 1024, 1025, 13*1024+17,
             3*1024+1000, 65*1024+5, then 245 uniform on [0, 2^20] (lengths seed 5); packed
             at 16-byte aligned offsets with at least 16 gap bytes of 0xA5 between messages
             (a kernel that reads past a message end hashes 0xA5s and fails parity);
             bytes seed 5, per-message keys seed 15
  fp32_8192  one keyed hash of an 8192 x 8192 float32 tensor of N(0,1) values (256 MiB,
             hashed as its little-endian storage bytes); values seed 2, key seed 12
  gib4       one keyed hash of 4 GiB + 1000 uniform bytes (4,194,305 chunks: a 1000-byte
             tail and a multi-level root reduction); bytes seed 3, key seed 13
  batch64k   65,536 keyed hashes of 64 KiB each, contiguous (4 GiB); bytes seed 4,
             per-message keys seed 14
  gib16      one keyed hash of 16 GiB + 777 uniform bytes (16,777,217 chunks; the deepest
             level chain); bytes seed 4 (fresh generator), key seed 14
"""
import torch

GIB = 1 << 30
RAGGED_FIXED = [0, 1, 63, 64, 65, 1023, 1024, 1025, 13 * 1024 + 17, 3 * 1024 + 1000, 65 * 1024 + 5]

SIZES = {
    "mib1": 1 << 20,
    "fp32_8192": 8192 * 8192 * 4,
    "gib4": 4 * GIB + 1000,
    "batch64k": 65536 * 65536,
    "gib16": 16 * GIB + 777,
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def random_bytes(n, seed, device):
    """n uniform random bytes as a uint8 tensor on `device`."""
    t = torch.empty(n, dtype=torch.uint8, device=device)
    if n:
        t.random_(0, 256, generator=_gen(seed, device))
    return t


def key_bytes(seed, count=1):
    """`count` 32-byte keys from a CPU generator, as a (count, 32) uint8 CPU tensor."""
    return torch.randint(0, 256, (count, 32), dtype=torch.uint8, generator=_gen(seed, "cpu"))


def ragged_lengths(seed=5, count=256, max_len=1 << 20):
    rest = torch.randint(0, max_len + 1, (count - len(RAGGED_FIXED),), dtype=torch.int64,
                         generator=_gen(seed, "cpu")).tolist()
    return RAGGED_FIXED + rest


def pack_messages(lengths, gap=16, align=16):
    """Byte offsets that lay messages out back to back, each start aligned to `align`,
    with at least `gap` bytes between consecutive messages; returns (offsets, total)."""
    offs, pos = [], 0
    for n in lengths:
        offs.append(pos)
        pos = (pos + n + gap + align - 1) // align * align
    return offs, pos


def ragged_batch(device, seed=5, key_seed=15, count=256, max_len=1 << 20):
    """(base, offsets, lengths, keys (n, 32) uint8 CPU) for the ragged workload."""
    lengths = ragged_lengths(seed, count, max_len)
    offs, total = pack_messages(lengths)
    base = torch.full((total,), 0xA5, dtype=torch.uint8, device=device)
    data = random_bytes(total, seed, device)
    for o, n in zip(offs, lengths):
        base[o:o + n] = data[o:o + n]
    return base, offs, lengths, key_bytes(key_seed, count)


def uniform_batch(count, msg_len, device, seed=4, key_seed=14):
    """count contiguous messages of msg_len bytes: (base, offsets, lengths, keys CPU)."""
    base = random_bytes(count * msg_len, seed, device)
    offs = [i * msg_len for i in range(count)]
    return base, offs, [msg_len] * count, key_bytes(key_seed, count)


def single(name, device):
    """(tensor, key (32,) uint8 CPU) for a single-message workload."""
    if name == "mib1":
        return random_bytes(SIZES[name], 0, device), key_bytes(1)[0]
    if name == "fp32_8192":
        t = torch.randn(8192, 8192, dtype=torch.float32, device=device, generator=_gen(2, device))
        return t, key_bytes(12)[0]
    if name == "gib4":
        return random_bytes(SIZES[name], 3, device), key_bytes(13)[0]
    if name == "gib16":
        return random_bytes(SIZES[name], 4, device), key_bytes(14)[0]
    raise KeyError(name)
