"""bench.py's contract checks that need no GPU: more than one GPU is refused with a message
and exit status 2, and the op-count helpers count compressions as the BLAKE3 tree has them."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_compression_counts():
    # a whole hash: every block of every chunk plus one parent per internal node (n - 1)
    assert bench.message_compressions(0) == 1
    assert bench.message_compressions(1) == 1
    assert bench.message_compressions(1024) == 16
    assert bench.message_compressions(1025) == 16 + 1 + 1
    assert bench.message_compressions(13 * 1024 + 17) == 13 * 16 + 1 + 13
    # the leaf pass: blocks plus the parents inside each workgroup (k chunks -> k - 1)
    assert bench.leaf_compressions(4 * 1024, 1024) == 64 + 3
    assert bench.leaf_compressions((1 << 32) + 1000, 1024) == (1 << 22) * 16 + 16 + (1 << 22) - (1 << 12)


def test_kernel_digest_ignores_comments(tmp_path):
    src = os.path.join(ROOT, "blake3_merkle_tree_amd", "csrc")
    for f in ("b3_device.h", "b3_kernels.hip", "b3_kernels.h"):
        text = open(os.path.join(src, f)).read()
        (tmp_path / f).write_text("// a comment\n" + text.replace("\n", "\n\n", 3) + "/* and another */\n")
    assert bench.kernel_source_digest(str(tmp_path)) == bench.kernel_source_digest()
    with open(tmp_path / "b3_kernels.hip", "a") as fh:
        fh.write("static int extra;\n")
    assert bench.kernel_source_digest(str(tmp_path)) != bench.kernel_source_digest()
