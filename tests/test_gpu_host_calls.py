"""Host behaviour of the library's calls on a GPU: growing a call's scratch never waits for
the device. Freeing device or pinned memory (hipFree, hipHostFree) waits for every stream of
the device, so memory a scratch slot or a pinned table buffer outgrows is kept instead; a
call that grows them while another stream is busy returns before that stream is done."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Run in a fresh process, so that the library's scratch slots start empty: four calls on four
# streams, each queued behind work on its stream, take one 1 MiB slot each; then, with another
# stream busy for tens of milliseconds and no library call on it, a batch of 65,536 messages
# of two lengths (a task table of more than 1 MiB) grows an idle slot and a pinned buffer.
SCRIPT = r"""
import json, sys, time
import numpy as np
import torch
sys.path.insert(0, ROOT)
import blake3_merkle_tree_amd as b3
dev = torch.device("cuda:0")
filler = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
small = torch.zeros((300 << 10) + 5, dtype=torch.uint8, device=dev)
lens = np.array([5000 + (i & 1) for i in range(65536)], dtype=np.uint64)
offs = np.arange(65536, dtype=np.uint64) * 5008
base = torch.zeros(65536 * 5008, dtype=torch.uint8, device=dev)
key = bytes(32)
torch.cuda.synchronize()
for s in [torch.cuda.Stream() for _ in range(4)]:
    with torch.cuda.stream(s):
        for _ in range(20):
            filler.fill_(1)
        b3.keyed_hash(small, key)
torch.cuda.synchronize()
busy = torch.cuda.Stream()
with torch.cuda.stream(busy):
    for _ in range(1000):
        filler.fill_(2)
t0 = time.perf_counter()
out = b3.keyed_hash_batch(base, offs, lens)
t1 = time.perf_counter()
busy_after = not busy.query()
torch.cuda.synchronize()
t2 = time.perf_counter()
print(json.dumps({"call_ms": 1e3 * (t1 - t0), "busy_after_call": busy_after, "wait_ms": 1e3 * (t2 - t1)}))
"""


def test_scratch_growth_does_not_wait_for_other_streams():
    print("fresh process: slot growth while another stream is busy", flush=True)
    r = subprocess.run([sys.executable, "-c", SCRIPT.replace("ROOT", repr(ROOT))], capture_output=True, text=True,
                       timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print(res, flush=True)
    assert res["busy_after_call"], res  # the call returned while the other stream still ran
