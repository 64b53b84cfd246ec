"""Register spills in the built kernels (host only: reads the gfx950 code objects).

A kernel that spills keeps part of its working set in scratch memory, which
turns the streaming kernel's in-register K/V ring into extra HBM traffic (a
dtype branch once did exactly that at head_dim 256, tripling its time). Every
kernel the library runs by default must therefore have no private segment. The
optional ring variants used for tuning sweeps (higher occupancy) are exempt.
"""
from __future__ import annotations

import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

from paged_gqa_decode_block_amd import LIB_PATH

READELF = shutil.which("llvm-readelf") or "/opt/rocm/llvm/bin/llvm-readelf"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# default ring variant per head_dim: (ring slots, waves per SIMD, Q' in LDS); at d = 256
# a pair of waves splits the head dims
DEFAULT_STREAM = {64: (6, 2, 0), 128: (3, 2, 0), 256: (2, 2, 0)}


def _private_segment_sizes(lib: str) -> dict[str, int]:
    """Kernel name -> private_segment_fixed_size from every gfx950 code object
    in the library's offload bundles."""
    data = open(lib, "rb").read()
    sizes: dict[str, int] = {}
    pos = 0
    while True:
        i = data.find(BUNDLE_MAGIC, pos)
        if i < 0:
            break
        pos = i + len(BUNDLE_MAGIC)
        (n,) = struct.unpack_from("<Q", data, pos)
        off = pos + 8
        for _ in range(n):
            o, s, ts = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + ts].decode()
            off += ts
            if "gfx950" not in triple:
                continue
            with tempfile.NamedTemporaryFile(suffix=".co", delete=False) as f:
                f.write(data[i + o:i + o + s])
                path = f.name
            try:
                notes = subprocess.run([READELF, "--notes", path], capture_output=True, text=True,
                                       check=True).stdout
            finally:
                os.unlink(path)
            name = None
            for line in notes.splitlines():
                m = re.search(r"\.name:\s+(\S+)", line)
                if m:
                    name = m.group(1)
                m = re.search(r"\.private_segment_fixed_size:\s+(\d+)", line)
                if m and name:
                    sizes[name] = int(m.group(1))
    return sizes


def _is_tuning_variant(name: str) -> bool:
    m = re.search(r"partition_stream_kernelI\w+?Li(\d+)ELi(\d+)ELi(\d+)ELi\d+ELb(\d)", name)
    if not m:
        return False
    d, nbuf, occ, ql = (int(x) for x in m.groups())
    return DEFAULT_STREAM.get(d) != (nbuf, occ, ql)


@pytest.mark.skipif(not os.path.exists(LIB_PATH), reason="library not built")
@pytest.mark.skipif(not os.path.exists(READELF), reason="llvm-readelf not available")
def test_default_kernels_do_not_spill():
    sizes = _private_segment_sizes(LIB_PATH)
    assert any("partition_stream_kernel" in k for k in sizes), "no streaming kernel found"
    assert any("combine_kernel" in k for k in sizes)
    spilled = {k: v for k, v in sizes.items() if v and not _is_tuning_variant(k)}
    assert not spilled, f"kernels with scratch (bytes per lane): {spilled}"
    # every default stream configuration is present, for both q/out dtypes
    for d, (nbuf, occ, ql) in DEFAULT_STREAM.items():
        for qo in (0, 1):
            pat = f"Li{d}ELi{nbuf}ELi{occ}ELi2ELb{ql}ELi{qo}E"
            assert any("partition_stream_kernel" in k and pat in k for k in sizes), pat
