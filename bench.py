"""Benchmark: keyed BLAKE3 of one device-resident buffer on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload gib4|gib16|fp32_8192|mib1|batch64k|ragged256|xof_gib8]

A step is one full hash (leaf pass + level passes, ROOT) of the workload's bytes, which
are already in HBM when the timed region starts. Prints ONE JSON line on stdout:
  value         input bytes / 1e9 / seconds per step (GB/s), whole job, one GPU
  roofline      the dominant kernel (the leaf pass: chunk compression + fused in-workgroup
                tree), timed alone with HIP events on the stream it runs on, against the
                integer-VALU peak (it is ALU-bound; the HBM figure is reported beside it)
  cpu_baseline  the CPU oracle on host threads over a bounded sample of the same bytes
Everything else goes to stderr.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s hashed, single keyed BLAKE3 of 4 GiB input; % of VALU/HBM roofline"

# Integer VALU peak of MI355X: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz
# = 39.32e12 32-bit lane operations per second (no packed 32-bit integer add exists).
VALU_INT_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
# VALU lane-ops per compression on gfx950: 7 rounds x 8 quarter-rounds x 12 (2 v_add3_u32,
# 2 v_add_u32, 4 v_xor_b32, 4 v_alignbit_b32) + 8 v_xor_b32 for the output fold. This is the
# algorithmic count the roofline uses; the leaf issues 676 for a block chained inside a
# chunk, whose fold merges into the next block's first round.
OPS_PER_COMPRESSION = 7 * 8 * 12 + 8
# The BLAKE3 page's own count, 7 rounds x 8 quarter-rounds x 6 ops = 336 per 64-byte block,
# i.e. 5.25 ops per input byte; it undercounts the quarter-round (12 VALU instructions on
# gfx950), and is reported beside the literal count only as the page defines it.
PAGE_OPS_PER_BYTE = 336 / 64
LEAF_LANES = 256
BATCH_COUNT, BATCH_LEN = 65536, 65536  # the batch workload: 65,536 messages of 64 KiB
CPU_SHARE = 16  # host threads of one GPU's share on the benchmark machines


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def leaf_compressions(length, group_chunks):
    """Compressions the leaf pass performs: every block of every chunk, plus the parents
    inside each workgroup (a workgroup of k chunks has k-1)."""
    if length == 0:
        return 1
    full, tail = divmod(length, 1024)
    blocks = full * 16 + (0 if tail == 0 else (tail + 63) // 64)
    n = full + (1 if tail else 0)
    groups = (n + group_chunks - 1) // group_chunks
    return blocks + (n - groups)


def message_compressions(length):
    """Compressions of one whole hash: every block of every chunk plus n - 1 parents."""
    if length == 0:
        return 1
    full, tail = divmod(length, 1024)
    n = full + (1 if tail else 0)
    return full * 16 + (0 if tail == 0 else (tail + 63) // 64) + n - 1


def kernel_source_digest(csrc=None):
    """Digest of the kernel sources with comments and whitespace runs removed: it changes
    when the device code does, not when a comment does."""
    csrc = csrc or os.path.join(ROOT, "blake3_merkle_tree_amd", "csrc")
    h = hashlib.sha256()
    for f in ("b3_device.h", "b3_kernels.hip", "b3_kernels.h"):
        with open(os.path.join(csrc, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per leaf launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"leaf_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


XOF_WORKLOAD = "xof_gib8"
# An output block keeps all 16 words: the 8 xors of the fold plus 8 more for v[i+8] ^ cv[i].
XOF_OPS_PER_BLOCK = 7 * 8 * 12 + 16
XOF_OUT_BYTES = 8 << 30
XOF_CHECK_BYTES = 64 << 20


def bench_xof(args, torch, b3, workloads, dev, stream):
    """Extendable output: 8 GiB of keyed XOF output from the 1 MiB input. The step is the
    whole call (the input's two top subtrees, then the expansion kernel, one lane per
    64-byte block); the expansion is the dominant kernel, and its roofline is taken over
    the step's time (the input hash, ~30 us, is included in the time, not in the ops)."""
    data, key_t = workloads.single("mib1", dev)
    key = bytes(key_t.tolist())
    out = torch.empty(XOF_OUT_BYTES, dtype=torch.uint8, device=dev)

    def step():
        b3.hash_xof(data, key, XOF_OUT_BYTES, out=out)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    value = XOF_OUT_BYTES / 1e9 / (ms / 1e3)
    ops = (XOF_OUT_BYTES // 64) * XOF_OPS_PER_BLOCK
    achieved = ops / (ms / 1e3) / 1e12
    log(f"xof: {ms:.4f} ms/step ({value:.1f} GB/s of output), {achieved:.2f} Tops/s = "
        f"{achieved / VALU_INT_PEAK_TOPS:.1%} of the int-VALU peak")
    cpu = None
    digest_match = None
    if not args.no_check or not args.no_cpu:
        import oracle
        host = data.contiguous().view(torch.uint8).reshape(-1).cpu().numpy()
        c0 = time.perf_counter()
        want = oracle.hash_xof(host, key, XOF_CHECK_BYTES)
        c_s = time.perf_counter() - c0
        if not args.no_cpu:
            cpu = {"value": round(XOF_CHECK_BYTES / 1e9 / c_s, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                   "sample": f"the first {XOF_CHECK_BYTES} bytes of the same output stream, plain scalar C "
                             f"oracle on one thread, {c_s:.2f} s wall"}
        if not args.no_check:
            digest_match = bytes(out[:XOF_CHECK_BYTES].cpu().numpy().tobytes()) == want
            log(f"first {XOF_CHECK_BYTES} output bytes match the oracle: {digest_match}")
    rec = {
        "metric": "GB/s of extended output, keyed BLAKE3 XOF",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u32", "data": "synthetic",
        "config": {"workload": "8 GiB of keyed BLAKE3 extendable output of 1 MiB uniform random bytes "
                               "(seed 0, key seed 1)", "input_bytes": data.numel(), "output_bytes": XOF_OUT_BYTES},
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_INT_PEAK_TOPS, 3),
                     "unit": "Tops/s (int32 VALU lane-ops)", "frac": round(achieved / VALU_INT_PEAK_TOPS, 4),
                     "traffic": None, "kernel": "xof_expand_kernel (step time, input hash included)",
                     "kernel_ms": round(ms, 4), "ops_per_launch": ops,
                     "hbm_write_gbs": round(value, 1), "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu,
        "digest_match": digest_match,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clock settles only after ~100 ms of this load: warm up past that
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="gib4")
    ap.add_argument("--cpu-sample-gib", type=float, default=None,
                    help="time the CPU oracle on the first GIB GiB only (default: the whole input)")
    ap.add_argument("--no-check", action="store_true", help="skip the full-digest oracle check")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--calibrate-copy", type=float, default=None, metavar="GIB",
                    help="only run an elementwise copy kernel over GIB GiB (reads and writes that many "
                         "bytes) --steps times: the reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the hash of one buffer "
              "runs on a single device, and sharding an input across devices is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import blake3_merkle_tree_amd as b3
    from blake3_merkle_tree_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy is not None:
        n = int(args.calibrate_copy * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "launches": args.steps}), flush=True)
        return
    if args.workload == XOF_WORKLOAD:
        return bench_xof(args, torch, b3, workloads, dev, stream)
    batch = args.workload in ("batch64k", "ragged256")
    if batch:
        if args.workload == "batch64k":
            base, offs, lengths, keys_cpu = workloads.uniform_batch(BATCH_COUNT, BATCH_LEN, dev)
        else:
            base, offs, lengths, keys_cpu = workloads.ragged_batch(dev)
        keys = keys_cpu.to(dev)
        nbytes = sum(lengths)
        out = torch.empty((len(lengths), 32), dtype=torch.uint8, device=dev)
        offs_np = np.asarray(offs, dtype=np.uint64)
        lens_np = np.asarray(lengths, dtype=np.uint64)

        def step():
            b3.keyed_hash_batch(base, offs_np, lens_np, keys, out=out)
        data = base
    else:
        data, key_t = workloads.single(args.workload, dev)
        key = bytes(key_t.tolist())
        nbytes = data.numel() * data.element_size()
        out = torch.empty(32, dtype=torch.uint8, device=dev)

        def step():
            b3.keyed_hash(data, key, out=out)
    torch.cuda.synchronize()
    log(f"workload {args.workload}: {nbytes} bytes")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    value = nbytes / 1e9 / (ms_per_step / 1e3)
    log(f"chain: {ms_per_step:.4f} ms/step ({value:.1f} GB/s), wall {wall:.3f} s for {args.steps} steps")

    # the dominant kernel alone: the leaf pass, launched on the same stream
    roofline = None
    if args.workload == "ragged256":
        # leaf and level launches over the task table: the roofline is taken over the step
        ops = sum(message_compressions(n) for n in lengths) * OPS_PER_COMPRESSION
        achieved = ops / (ms_per_step / 1e3) / 1e12
        roofline = {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": round(VALU_INT_PEAK_TOPS, 3),
            "unit": "Tops/s (int32 VALU lane-ops)",
            "frac": round(achieved / VALU_INT_PEAK_TOPS, 4),
            "traffic": None,
            "kernel": "whole step (leaf_batch_kernel + level_batch_kernel launches, task table upload)",
            "kernel_ms": round(ms_per_step, 4),
            "ops_per_launch": ops,
            "hbm_gbs": round(value, 1),
            "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        }
        log(f"step (all kernels): {achieved:.2f} Tops/s = {achieved / VALU_INT_PEAK_TOPS:.1%} of the int-VALU peak")
    elif batch:
        # every 64 KiB message fits one leaf workgroup: the step is the leaf kernel alone,
        # one launch, so the chain's event timing is the kernel's
        k = b3.leaf_group_chunks(nbytes) // LEAF_LANES
        c = (BATCH_LEN + 1023) // 1024
        per_wg = LEAF_LANES // (1 << ((c + k - 1) // k - 1).bit_length())
        ops = BATCH_COUNT * leaf_compressions(BATCH_LEN, 1 << 40) * OPS_PER_COMPRESSION
        achieved = ops / (ms_per_step / 1e3) / 1e12
        roofline = {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": round(VALU_INT_PEAK_TOPS, 3),
            "unit": "Tops/s (int32 VALU lane-ops)",
            "frac": round(achieved / VALU_INT_PEAK_TOPS, 4),
            "traffic": measured_traffic(args.workload),
            "kernel": f"leaf_uniform_kernel<{k}> ({c} chunks per message, {per_wg} messages per workgroup)",
            "kernel_ms": round(ms_per_step, 4),
            "ops_per_launch": ops,
            "hbm_gbs": round(value, 1),
            "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        }
        log(f"leaf kernel (whole batch): {achieved:.2f} Tops/s = {achieved / VALU_INT_PEAK_TOPS:.1%} "
            "of the int-VALU peak")
    else:
        group = b3.leaf_group_chunks(nbytes)  # the leaf configuration the chain uses
        cvs = torch.empty(((nbytes + 1023) // 1024 + group - 1) // group, 8, dtype=torch.int32, device=dev)
        for _ in range(args.warmup):
            b3.group_cvs(data, key, group_chunks=group, out=cvs)
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        k0.record(stream)
        for _ in range(args.steps):
            b3.group_cvs(data, key, group_chunks=group, out=cvs)
        k1.record(stream)
        torch.cuda.synchronize()
        leaf_ms = k0.elapsed_time(k1) / args.steps
        ops = leaf_compressions(nbytes, group) * OPS_PER_COMPRESSION
        achieved = ops / (leaf_ms / 1e3) / 1e12
        roofline = {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": round(VALU_INT_PEAK_TOPS, 3),
            "unit": "Tops/s (int32 VALU lane-ops)",
            "frac": round(achieved / VALU_INT_PEAK_TOPS, 4),
            "traffic": measured_traffic(args.workload),
            "kernel": "leaf_quad_kernel" if group < LEAF_LANES else f"leaf_uniform_kernel<{group // LEAF_LANES}>",
            "kernel_ms": round(leaf_ms, 4),
            "ops_per_launch": ops,
            "hbm_gbs": round(nbytes / 1e9 / (leaf_ms / 1e3), 1),
            "hbm_frac": round(nbytes / 1e9 / (leaf_ms / 1e3) / HBM_PEAK_GBS, 4),
        }
        log(f"leaf kernel: {leaf_ms:.4f} ms, {achieved:.2f} Tops/s = {achieved / VALU_INT_PEAK_TOPS:.1%} "
            f"of the int-VALU peak; {nbytes / 1e9 / (leaf_ms / 1e3):.0f} GB/s")

    digest_match = None
    cpu = None
    if not args.no_check or not args.no_cpu:
        import oracle
        cores = min(CPU_SHARE, os.cpu_count() or 1)
        host = data.contiguous().view(torch.uint8).reshape(-1).cpu().numpy()
        want = None
        if not args.no_cpu:
            # the oracle over the whole input (or the first --cpu-sample-gib GiB of it)
            sample = len(host) if args.cpu_sample_gib is None else min(len(host), int(args.cpu_sample_gib * (1 << 30)))
            c0 = time.perf_counter()
            if batch:
                # whole messages from the front of the batch, until the sample's bytes are used
                cnt, end = 0, 0
                while cnt < len(lengths) and offs[cnt] + lengths[cnt] <= sample:
                    end = offs[cnt] + lengths[cnt]
                    cnt += 1
                got = oracle.hash_batch(host[:end], offs[:cnt], lengths[:cnt],
                                        keys_cpu.numpy().tobytes()[:32 * cnt], nthreads=cores)
                sample = sum(lengths[:cnt])
                if cnt < len(lengths):
                    got = None
            else:
                got = oracle.hash_mt(host[:sample], key, cores)
            c_s = time.perf_counter() - c0
            if got is not None and (batch or sample == len(host)):
                want = got
            what = "all" if want is not None else f"the first {sample}"
            cpu = {"value": round(sample / 1e9 / c_s, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
                   "sample": f"{what} bytes of the same {args.workload} input ({sample} B), plain scalar C oracle "
                             f"(multi-threaded aligned-subtree form), {c_s:.2f} s wall, {cores} threads"}
            log(f"cpu oracle: {cpu['value']} GB/s on {cores} threads ({sample} bytes)")
        if not args.no_check:
            if batch:
                if want is None:
                    want = oracle.hash_batch(host, offs, lengths, keys_cpu.numpy().tobytes(), nthreads=cores)
                digest_match = [bytes(r) for r in out.cpu().numpy()] == want
            else:
                if want is None:
                    want = oracle.hash_mt(host, key, cores)
                digest_match = bytes(out.cpu().tolist()) == want
            log(f"digest matches the oracle: {digest_match}")

    cfg = {
        "workload": {
            "gib4": "one keyed BLAKE3 of 4 GiB + 1000 uniform random bytes (seed 3, key seed 13)",
            "gib16": "one keyed BLAKE3 of 16 GiB + 777 uniform random bytes (seed 4, key seed 14)",
            "fp32_8192": "one keyed BLAKE3 of an 8192x8192 fp32 N(0,1) tensor's bytes (seed 2, key seed 12)",
            "mib1": "one keyed BLAKE3 of 1 MiB uniform random bytes (seed 0, key seed 1)",
            "batch64k": "65,536 keyed BLAKE3 hashes of 64 KiB each (seed 4, key seed 14)",
            "ragged256": "256 keyed BLAKE3 hashes of ragged lengths 0 B .. 1 MiB (lengths and bytes seed 5, "
                         "key seed 15), packed with 0xA5 gaps",
        }[args.workload],
        "bytes": nbytes,
        "chunks": (nbytes + 1023) // 1024,
        "leaf_workgroup_chunks": b3.leaf_group_chunks(nbytes),
        "level_workgroup_cvs": 256,
    }
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": cfg,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "digest_match": digest_match,
        "hbm_frac_chain": round(value / HBM_PEAK_GBS, 4),
        "roof_at_page_op_count": {
            "ops_per_byte": PAGE_OPS_PER_BYTE,
            "roof_gbs": round(min(HBM_PEAK_GBS, VALU_INT_PEAK_TOPS * 1e3 / PAGE_OPS_PER_BYTE), 1),
            "frac": round(value / min(HBM_PEAK_GBS, VALU_INT_PEAK_TOPS * 1e3 / PAGE_OPS_PER_BYTE), 4),
        },
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
