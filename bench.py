"""Benchmark: keyed BLAKE3 of one device-resident buffer on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload gib4|gib16|fp32_8192|mib1|batch64k|ragged256|xof_gib8]

A step is one full hash (leaf pass + level passes, ROOT) of the workload's bytes, which
are already in HBM when the timed region starts. Before the W counted warm-up steps the
step runs for --warmup-seconds of wall time (the GPU's clock and power settle only after
~100 ms of this load). The K timed steps run back to back on one stream with a HIP event
between consecutive steps. Prints ONE JSON line on stdout:
  value         input bytes / 1e9 / median seconds per step (GB/s), whole job, one GPU
  ms_per_step   the median step; ms_per_step_min and ms_per_step_mean beside it, and
                ms_per_step_back_to_back: K more steps with no event between them
  roofline      the dominant kernel (the leaf pass: chunk compression + fused in-workgroup
                tree), timed alone with HIP events on the stream it runs on, each launch
                alternating with a whole step so that it runs in the chain's clock and
                power state (median launch), against the integer-VALU peak (it is
                ALU-bound; the HBM figure is reported beside it)
  gpu_state     gfx clock, temperatures and power read from the GPU's sysfs files while
                the timed steps ran
  cpu_baseline  the CPU oracle on the host's threads over the same bytes, plus one thread
                on a bounded sample, with the CPU model
Everything else goes to stderr.
"""
import argparse
import glob
import hashlib
import json
import os
import re
import statistics
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
ONE_THREAD_SAMPLE = 1 << 30  # bytes the one-thread oracle leg hashes (about 3 s)


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


def traffic_source(workload):
    return os.path.join("profiles", f"leaf_{workload}_traffic.txt")


def measured_traffic(workload):
    """HBM bytes per leaf launch from the committed rocprofv3 counter summary (taken in an
    earlier run, not in this one), if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, traffic_source(workload))
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


def host_cpu():
    """Threads this process may run on (what `nproc` prints), the machine's CPU count and
    the CPU model, from /proc/cpuinfo."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return {"nproc": nproc, "cpu_count": os.cpu_count(), "cpu_model": model}


class GpuSensors:
    """The benchmark GPU's gfx clock, temperatures and power, read from the amdgpu driver's
    sysfs files of its PCI device (hwmon freq1_input / temp*_input / power1_*, and the
    current pp_dpm_sclk level). Files only: no tool is started from this process."""

    def __init__(self, torch, index):
        self.dir = None
        self.hwmon = []
        try:
            p = torch.cuda.get_device_properties(index)
            d = f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
            if os.path.isdir(d):
                self.dir = d
                self.hwmon = sorted(glob.glob(os.path.join(d, "hwmon", "hwmon*")))
        except Exception:  # noqa: BLE001 - sensors are optional
            pass

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            return None

    def sample(self):
        s = {}
        for h in self.hwmon:
            for f in glob.glob(os.path.join(h, "freq*_input")):
                label = self._read(f.replace("_input", "_label")) or os.path.basename(f)
                v = self._read(f)
                if v is not None and v.isdigit():
                    s[f"{label}_mhz"] = int(v) / 1e6
            for f in glob.glob(os.path.join(h, "temp*_input")):
                label = self._read(f.replace("_input", "_label")) or os.path.basename(f)
                v = self._read(f)
                if v is not None and v.lstrip("-").isdigit():
                    s[f"temp_{label}_c"] = int(v) / 1e3
            for name in ("power1_average", "power1_input"):
                v = self._read(os.path.join(h, name))
                if v is not None and v.isdigit():
                    s[f"{name}_w"] = int(v) / 1e6
        if self.dir:
            levels = self._read(os.path.join(self.dir, "pp_dpm_sclk"))
            if levels:
                cur = [ln for ln in levels.splitlines() if ln.rstrip().endswith("*")]
                if cur:
                    m = re.search(r"(\d+)\s*[Mm]hz", cur[0])
                    if m:
                        s["pp_dpm_sclk_mhz"] = int(m.group(1))
        return s

    def summary(self, samples):
        """Median, minimum and maximum of every sampled quantity."""
        if not samples:
            return {"source": self.dir, "samples": 0}
        out = {"source": self.dir, "samples": len(samples)}
        for k in sorted({k for smp in samples for k in smp}):
            v = [smp[k] for smp in samples if k in smp]
            out[k] = {"median": round(statistics.median(v), 1), "min": round(min(v), 1), "max": round(max(v), 1)}
        return out


def warm_up(torch, step, seconds, count, depth=0):
    """Runs `step` for at least `seconds` of wall time (synchronising every few steps, so
    that the time is the GPU's), then `count` more steps. Those go back to back without a
    synchronisation, at least `depth` of them (the timed loop's length): calls queued that
    deep make the library grow its per-call resources (scratch from the stream-ordered pool,
    pinned table buffers) once, and that growth belongs to the warm-up, not to a timed step."""
    t_end = time.perf_counter() + seconds
    n = 0
    while True:
        for _ in range(4):
            step()
        n += 4
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    count = max(count, depth)
    for _ in range(count):
        step()
    torch.cuda.synchronize()
    return n + count


def timed_steps(torch, stream, step, k, sensors=None):
    """Runs `step` k times back to back on `stream`, a HIP event recorded before the first
    and after every step; while they run, samples the GPU's sensors. Returns the per-step
    times (ms), the event time of all k steps (ms), the host wall time (s) and the samples."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(k):
        step()
        evs[i + 1].record(stream)
    samples = []
    if sensors is not None:
        while not evs[k].query():
            samples.append(sensors.sample())
            time.sleep(0.002)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(k)]
    return per, evs[0].elapsed_time(evs[k]), wall, samples


def timed_pairs(torch, stream, a, b, k):
    """k pairs (a, b) back to back on `stream`, HIP events around every `a`: the times of
    the a's (ms), each run in the clock and power state that alternating with b sets."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * k)]
    torch.cuda.synchronize()
    for i in range(k):
        evs[2 * i].record(stream)
        a()
        evs[2 * i + 1].record(stream)
        b()
    torch.cuda.synchronize()
    return [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(k)]


def back_to_back(torch, stream, step, k):
    """Mean time (ms) of k steps with no event between them."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(k):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / k


def step_stats(per, total, k):
    return {"median": statistics.median(per), "min": min(per), "mean": total / k}


XOF_WORKLOAD = "xof_gib8"
# An output block keeps all 16 words: the 8 xors of the fold plus 8 more for v[i+8] ^ cv[i].
XOF_OPS_PER_BLOCK = 7 * 8 * 12 + 16
XOF_OUT_BYTES = 8 << 30
XOF_CHECK_BYTES = 64 << 20


def oracle_threads(cpu):
    """Threads of the multi-threaded oracle leg: every thread this process may run on, up
    to one GPU's host share on the benchmark machines."""
    return max(1, min(cpu["nproc"], CPU_SHARE))


def bench_xof(args, torch, b3, workloads, dev, stream, sensors):
    """Extendable output: 8 GiB of keyed XOF output from the 1 MiB input. The step is the
    whole call (the input's two top subtrees, then the expansion kernel, one lane per
    64-byte block); the expansion is the dominant kernel, and its roofline is taken over
    the step's time (the input hash, ~30 us, is included in the time, not in the ops)."""
    data, key_t = workloads.single("mib1", dev)
    key = bytes(key_t.tolist())
    out = torch.empty(XOF_OUT_BYTES, dtype=torch.uint8, device=dev)

    def step():
        b3.hash_xof(data, key, XOF_OUT_BYTES, out=out)
    warm = warm_up(torch, step, args.warmup_seconds, args.warmup, args.steps)
    per, total, wall, samples = timed_steps(torch, stream, step, args.steps, sensors)
    st = step_stats(per, total, args.steps)
    ms = st["median"]
    value = XOF_OUT_BYTES / 1e9 / (ms / 1e3)
    ops = (XOF_OUT_BYTES // 64) * XOF_OPS_PER_BLOCK
    achieved = ops / (ms / 1e3) / 1e12
    log(f"xof: {ms:.4f} ms/step median (min {st['min']:.4f}, mean {st['mean']:.4f}; {value:.1f} GB/s of "
        f"output), {achieved:.2f} Tops/s = {achieved / VALU_INT_PEAK_TOPS:.1%} of the int-VALU peak")
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
                             f"oracle on one thread (its extended output has no multi-threaded form), "
                             f"{c_s:.2f} s wall", **host_cpu()}
        if not args.no_check:
            digest_match = bytes(out[:XOF_CHECK_BYTES].cpu().numpy().tobytes()) == want
            log(f"first {XOF_CHECK_BYTES} output bytes match the oracle: {digest_match}")
    rec = {
        "metric": "GB/s of extended output, keyed BLAKE3 XOF",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "ms_per_step_min": round(st["min"], 4), "ms_per_step_mean": round(st["mean"], 4),
        "warmup_steps_run": warm, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u32", "data": "synthetic",
        "config": {"workload": "8 GiB of keyed BLAKE3 extendable output of 1 MiB uniform random bytes "
                               "(seed 0, key seed 1)", "input_bytes": data.numel(), "output_bytes": XOF_OUT_BYTES},
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_INT_PEAK_TOPS, 3),
                     "unit": "Tops/s (int32 VALU lane-ops)", "frac": round(achieved / VALU_INT_PEAK_TOPS, 4),
                     "traffic": None, "kernel": "xof_expand_kernel (step time, input hash included)",
                     "kernel_ms": round(ms, 4), "ops_per_launch": ops,
                     "hbm_write_gbs": round(value, 1), "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "gpu_state": sensors.summary(samples),
        "cpu_baseline": cpu,
        "digest_match": digest_match,
    }
    print(json.dumps(rec), flush=True)


def cpu_legs(args, oracle, host, key, batch, cpu_info):
    """The oracle on the host: every byte with oracle_threads() threads (its digests are
    the check's expected values when it covers the whole input), and one thread on the
    first ONE_THREAD_SAMPLE bytes. Returns (cpu_baseline dict, expected digest(s) or None)."""
    threads = oracle_threads(cpu_info)
    sample = len(host) if args.cpu_sample_gib is None else min(len(host), int(args.cpu_sample_gib * (1 << 30)))

    def run(limit, nthreads):
        c0 = time.perf_counter()
        if batch is not None:
            offs, lengths, keys_bytes = batch
            # whole messages from the front of the batch, until the sample's bytes are used
            cnt = 0
            while cnt < len(lengths) and offs[cnt] + lengths[cnt] <= limit:
                cnt += 1
            end = offs[cnt - 1] + lengths[cnt - 1] if cnt else 0
            got = oracle.hash_batch(host[:end], offs[:cnt], lengths[:cnt], keys_bytes[:32 * cnt], nthreads=nthreads)
            nbytes = sum(lengths[:cnt])
            whole = cnt == len(lengths)
        else:
            got = oracle.hash_mt(host[:limit], key, nthreads)  # one thread too: the same aligned-subtree form
            nbytes = limit
            whole = limit == len(host)
        return nbytes / 1e9 / (time.perf_counter() - c0), nbytes, (got if whole else None), time.perf_counter() - c0

    rate, nbytes, want, secs = run(sample, threads)
    what = "all" if want is not None else f"the first {nbytes}"
    one_rate, one_bytes, one_want, one_secs = run(min(len(host), ONE_THREAD_SAMPLE), 1)
    if want is None:
        want = one_want
    cpu = {"value": round(rate, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{what} bytes of the same {args.workload} input ({nbytes} B), plain scalar C oracle "
                     f"(multi-threaded aligned-subtree form), {secs:.2f} s wall, {threads} threads",
           "one_thread": {"value": round(one_rate, 3), "unit": "GB/s",
                          "sample": f"the first {one_bytes} bytes of the same input, the same oracle form on one "
                                    f"thread, {one_secs:.2f} s wall"},
           **cpu_info}
    log(f"cpu oracle: {cpu['value']} GB/s on {threads} threads ({nbytes} bytes); {cpu['one_thread']['value']} "
        f"GB/s on one thread ({one_bytes} bytes); nproc {cpu_info['nproc']}, {cpu_info['cpu_model']}")
    return cpu, want


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10, help="counted warm-up steps, after --warmup-seconds")
    # the GPU's clock and power settle only after ~100 ms of this load: warm up past that
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="wall time of untimed steps before the counted warm-up")
    ap.add_argument("--workload", default="gib4")
    ap.add_argument("--cpu-sample-gib", type=float, default=None,
                    help="time the multi-threaded CPU oracle on the first GIB GiB only (default: the whole input)")
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
    sensors = GpuSensors(torch, 0)
    if args.workload == XOF_WORKLOAD:
        return bench_xof(args, torch, b3, workloads, dev, stream, sensors)
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

    warm = warm_up(torch, step, args.warmup_seconds, args.warmup, args.steps)
    per, total, wall, samples = timed_steps(torch, stream, step, args.steps, sensors)
    st = step_stats(per, total, args.steps)
    ms_per_step = st["median"]
    value = nbytes / 1e9 / (ms_per_step / 1e3)
    log(f"chain: {ms_per_step:.4f} ms/step median, min {st['min']:.4f}, mean {st['mean']:.4f} ({value:.1f} GB/s); "
        f"wall {wall:.3f} s for {args.steps} steps after {warm} warm-up steps")
    gpu_state = sensors.summary(samples)
    log(f"gpu state during the timed steps: {gpu_state}")
    b2b = back_to_back(torch, stream, step, args.steps)
    log(f"the same steps with no event between them: {b2b:.4f} ms/step")

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
            "kernel": "whole step (task-table upload, batch leaf and level passes)",
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
            "traffic_source": traffic_source(args.workload) + " (rocprofv3 counters of an earlier run)",
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

        def leaf_step():
            b3.group_cvs(data, key, group_chunks=group, out=cvs)
        # each leaf launch alternates with a whole step, so that it runs in the clock and
        # power state of the chain
        leaf_step()
        kper = timed_pairs(torch, stream, leaf_step, step, args.steps)
        kst = step_stats(kper, sum(kper), args.steps)
        leaf_ms = kst["median"]
        ops = leaf_compressions(nbytes, group) * OPS_PER_COMPRESSION
        achieved = ops / (leaf_ms / 1e3) / 1e12
        roofline = {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": round(VALU_INT_PEAK_TOPS, 3),
            "unit": "Tops/s (int32 VALU lane-ops)",
            "frac": round(achieved / VALU_INT_PEAK_TOPS, 4),
            "traffic": measured_traffic(args.workload),
            "traffic_source": traffic_source(args.workload) + " (rocprofv3 counters of an earlier run)",
            "kernel": "leaf_quad_kernel" if group < LEAF_LANES else f"leaf_uniform_kernel<{group // LEAF_LANES}>",
            "kernel_ms": round(leaf_ms, 4),
            "kernel_ms_min": round(kst["min"], 4),
            "kernel_ms_mean": round(kst["mean"], 4),
            "ops_per_launch": ops,
            "hbm_gbs": round(nbytes / 1e9 / (leaf_ms / 1e3), 1),
            "hbm_frac": round(nbytes / 1e9 / (leaf_ms / 1e3) / HBM_PEAK_GBS, 4),
        }
        log(f"leaf kernel: {leaf_ms:.4f} ms median (min {kst['min']:.4f}), {achieved:.2f} Tops/s = "
            f"{achieved / VALU_INT_PEAK_TOPS:.1%} of the int-VALU peak; {nbytes / 1e9 / (leaf_ms / 1e3):.0f} GB/s")

    digest_match = None
    cpu = None
    if not args.no_check or not args.no_cpu:
        import oracle
        cpu_info = host_cpu()
        host = data.contiguous().view(torch.uint8).reshape(-1).cpu().numpy()
        bspec = (offs, lengths, keys_cpu.numpy().tobytes()) if batch else None
        want = None
        if not args.no_cpu:
            cpu, want = cpu_legs(args, oracle, host, None if batch else key, bspec, cpu_info)
        if not args.no_check:
            threads = oracle_threads(cpu_info)
            if batch:
                if want is None:
                    want = oracle.hash_batch(host, offs, lengths, bspec[2], nthreads=threads)
                digest_match = [bytes(r) for r in out.cpu().numpy()] == want
            else:
                if want is None:
                    want = oracle.hash_mt(host, key, threads)
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
    roof_page = min(HBM_PEAK_GBS, VALU_INT_PEAK_TOPS * 1e3 / PAGE_OPS_PER_BYTE)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_min": round(st["min"], 4),
        "ms_per_step_mean": round(st["mean"], 4),
        "ms_per_step_back_to_back": round(b2b, 4),
        "warmup_steps_run": warm,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": cfg,
        "roofline": roofline,
        "gpu_state": gpu_state,
        "cpu_baseline": cpu,
        "digest_match": digest_match,
        "hbm_frac_chain": round(value / HBM_PEAK_GBS, 4),
        "roof_at_page_op_count": {
            "ops_per_byte": PAGE_OPS_PER_BYTE,
            "roof_gbs": round(roof_page, 1),
            "frac": round(value / roof_page, 4),
        },
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
