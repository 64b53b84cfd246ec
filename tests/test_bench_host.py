"""Host-side checks of the benchmark's plumbing (no GPU needed)."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

CSRC = os.path.join(ROOT, "paged_gqa_decode_block_amd", "csrc")


def _local_includes(path):
    """Files of csrc/ that `path` includes, directly or through each other."""
    seen, todo = set(), [path]
    while todo:
        f = todo.pop()
        for inc in re.findall(r'#include\s+"([^"]+)"', open(f).read()):
            p = os.path.normpath(os.path.join(os.path.dirname(f), inc))
            if p.startswith(CSRC) and p not in seen:
                seen.add(p)
                todo.append(p)
    return seen


def test_kernel_hash_covers_the_streaming_kernel_and_its_headers():
    """HBM counter readings are reported only while this hash matches the one
    stored with them, so it must change with every file the streaming kernel
    is built from and with the launch code."""
    hashed = {os.path.normpath(os.path.join(ROOT, f)) for f in bench.KERNEL_SOURCES}
    stream = os.path.join(CSRC, "pa_partition_stream.hip")
    assert stream in hashed
    assert os.path.join(CSRC, "pa_api.hip") in hashed
    missing = _local_includes(stream) - hashed
    assert not missing, f"not hashed: {sorted(missing)}"


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
