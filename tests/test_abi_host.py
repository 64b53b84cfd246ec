"""The C ABI on the host: the library loads, exports what the header declares, the
ctypes descriptor matches the C struct, and every argument error is returned
before any device work (these tests never touch a GPU)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from paged_gqa_decode_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")


def _header_functions():
    """Every function declared in include/*.h."""
    names = set()
    for h in sorted(os.listdir(os.path.dirname(HEADER))):
        if h.endswith(".h"):
            text = open(os.path.join(os.path.dirname(HEADER), h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(paged_attn_\w+)\s*\(", text))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    lib = pa.load_library()
    declared = _header_functions()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    assert lib.paged_attn_abi_version() == 5


def test_descriptor_layout_matches_c(tmp_path):
    fields = [f for f, _ in pa.PaDesc._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "paged_attn.h"\n'
        "int main(void) { printf(\"%zu\", sizeof(pa_desc));\n"
        + "".join(f'  printf(" %zu", offsetof(pa_desc, {f}));\n' for f in fields)
        + "  return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(pa.PaDesc)] + [getattr(pa.PaDesc, f).offset for f in fields]
    assert got == want


def _desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, num_blocks=64,
                max_blocks_per_seq=16, kv_dtype="bf16", k_strides=(2 * 16 * 128, 16 * 128, 128),
                partition_size=0, path="auto")
    base.update(kw)
    return pa.make_desc(**base)


def test_valid_descriptor_and_resolved_path():
    assert pa.validate(_desc()) == 0
    # below 160 MB of K/V (by the max_blocks_per_seq bound) the grid kernel; at
    # and above it the streaming kernel, where it applies
    big = dict(max_blocks_per_seq=5120, num_blocks=16384)   # 2 * 2 * 81920 * 128 * 2 * 2 B = 160 MiB
    assert pa.PATH_NAME[pa.resolved_path(_desc())] == "mfma_grid"
    assert pa.PATH_NAME[pa.resolved_path(_desc(path="mfma"))] == "mfma_grid"
    assert pa.PATH_NAME[pa.resolved_path(_desc(path="mfma_stream"))] == "mfma_stream"
    assert pa.PATH_NAME[pa.resolved_path(_desc(**big))] == "mfma_stream"
    assert pa.PATH_NAME[pa.resolved_path(_desc(path="mfma", **big))] == "mfma_stream"
    assert pa.PATH_NAME[pa.resolved_path(_desc(max_blocks_per_seq=5119, num_blocks=16384))] == "mfma_grid"
    assert pa.PATH_NAME[pa.resolved_path(_desc(path="mfma_grid", **big))] == "mfma_grid"
    # the streaming kernel needs block_size >= 16 and at most 1024 sequences
    assert pa.PATH_NAME[pa.resolved_path(_desc(block_size=8, max_blocks_per_seq=16384, num_blocks=32768,
                                               k_strides=(2048, 1024, 128)))] == "mfma_grid"
    assert pa.PATH_NAME[pa.resolved_path(_desc(batch=1025, **big))] == "mfma_grid"
    assert pa.PATH_NAME[pa.resolved_path(_desc(kv_dtype="f32", k_strides=(4096, 2048, 128)))] == "valu"
    assert pa.PATH_NAME[pa.resolved_path(_desc(path="valu"))] == "valu"


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=7), -2),                 # H_q % H_kv
    (dict(batch=-1), -2),
    (dict(num_blocks=0), -2),
    (dict(head_dim=96), -3),
    (dict(block_size=24), -4),
    (dict(block_size=2048), -4),
    (dict(kv_dtype=7), -5),
    (dict(k_strides=(4096, 2048, 100)), -6),   # token stride < head_dim
    (dict(k_strides=(4096, 2048, 132)), -6),   # not a multiple of 16 bytes
    (dict(k_strides=(0, 2048, 128)), -6),
    (dict(partition_size=48), -8),
    (dict(partition_size=16), -8),
    (dict(partition_size=32768), -8),
    (dict(block_size=1, partition_size=2048), -8),  # spans more than the block-id table
    (dict(path=9), -10),
    (dict(path=6), -10),
    (dict(kv_dtype="f32", k_strides=(4096, 2048, 128), path="mfma_fused"), -10),
    # the merged grid variant's LDS bound: 2 * 32 partitions * G 16 + 16 > 16 * 64
    (dict(head_dim=64, k_strides=(2048, 1024, 64), num_q_heads=32, max_blocks_per_seq=64,
          partition_size=32, path="mfma_fused"), -8),
    (dict(kv_dtype="f32", k_strides=(4096, 2048, 128), path="mfma"), -10),
    (dict(kv_dtype="f32", k_strides=(4096, 2048, 128), path="mfma_stream"), -10),
    (dict(block_size=8, k_strides=(2048, 1024, 128), path="mfma_stream"), -10),
    (dict(batch=2000, path="mfma_stream"), -10),
    (dict(num_q_heads=2 * 12, path="valu"), -2),   # G = 12 beyond the VALU path
    (dict(num_q_heads=2 * 17), -2),                # G = 17 beyond every path
])
def test_descriptor_errors(kw, code):
    d = _desc(**kw)
    assert pa.validate(d) == code
    assert pa.workspace_size(d) == 0
    assert pa.strerror(code) not in ("", "unknown status")


def _al(x):
    return (x + 255) // 256 * 256


def _stream_waves(d, cus=256, occ=2, min_chunks=16):
    """Grid of the streaming kernel for head_dim 128 (two waves per SIMD): one
    wave per SIMD slot, fewer when the chunk bound gives each wave less than 16
    chunks, kept a multiple of the compute units while one per unit remains.
    (Without a GPU the library assumes 256 compute units.)"""
    bound = d.batch * d.num_kv_heads * ((d.max_blocks_per_seq * d.block_size + 15) // 16)
    grid = 4 * occ * cus
    w = bound // min_chunks
    if w >= grid:
        return grid
    if w >= cus:
        w = w // cus * cus
    return max(w, 1)


def test_partition_size_choice_and_workspace():
    # kernels with one workgroup per partition: nothing when one partition suffices
    d = _desc(partition_size=512, path="mfma_grid")
    assert pa.partition_size(d) == 512
    assert pa.workspace_size(d) == 0        # pmax = ceil(16*16 / 512) = 1
    d = _desc(partition_size=64, path="mfma_grid")
    pmax = 256 // 64
    rows = 2 * 8 * pmax
    assert pa.workspace_size(d) == 2 * _al(rows * 4) + _al(rows * 128 * 4)
    # the merged grid variant: arrival counters first (offset 0), then the states;
    # nothing when one partition suffices; resolved as asked
    d = _desc(partition_size=64, path="mfma_fused")
    assert pa.PATH_NAME[pa.resolved_path(d)] == "mfma_fused"
    assert pa.workspace_size(d) == _al(2 * 2 * 4) + 2 * _al(rows * 4) + _al(rows * 128 * 4)
    assert pa.workspace_size(_desc(partition_size=512, path="mfma_fused")) == 0
    # the LDS bound at its edge: 2 * 32 * 16 + 16 = 1040 > 1024, 2 * 31 * 16 + 16 = 1008
    edge = dict(head_dim=64, k_strides=(2048, 1024, 64), num_q_heads=32, partition_size=32,
                path="mfma_fused")
    assert pa.validate(_desc(max_blocks_per_seq=62, **edge)) == 0
    assert pa.validate(_desc(max_blocks_per_seq=64, **edge)) == -8
    # automatic partition of the merged variant: 1024, halved while the grid is
    # small but not below min(1024, max_tokens / 16), doubled to fit the LDS bound
    fz = dict(path="mfma_fused", partition_size=0)
    assert pa.partition_size(_desc(batch=8, num_q_heads=14, num_kv_heads=2, head_dim=64,
                                   k_strides=(2048, 1024, 64), max_blocks_per_seq=256, **fz)) == 256
    assert pa.partition_size(_desc(batch=64, num_q_heads=64, num_kv_heads=8,
                                   k_strides=(16 * 16 * 128, 16 * 128, 128),
                                   max_blocks_per_seq=2048, **fz)) == 1024
    assert pa.partition_size(_desc(max_blocks_per_seq=4, **fz)) == 64   # 64 tokens
    # 1 x 4 heads, 100000 tokens: 1024 is the floor; G = 16 at d = 64 needs more
    assert pa.partition_size(_desc(batch=1, num_q_heads=24, num_kv_heads=4, head_dim=256,
                                   k_strides=(4 * 16 * 256, 16 * 256, 256),
                                   max_blocks_per_seq=6250, **fz)) == 1024
    assert pa.partition_size(_desc(batch=1, num_q_heads=32, num_kv_heads=2, head_dim=64,
                                   k_strides=(2048, 1024, 64), max_blocks_per_seq=6250,
                                   **fz)) == 4096
    # the streaming kernel: a record (two int32) per (sequence, KV head) stream
    # and two state slots (max, sum, output of the G = 4 heads) per wave; the
    # partition size does not change it
    for part, mbs, batch in ((512, 16, 2), (64, 16, 2), (512, 2048, 64)):
        d = _desc(partition_size=part, max_blocks_per_seq=mbs, batch=batch, path="mfma_stream")
        assert pa.PATH_NAME[pa.resolved_path(d)] == "mfma_stream"
        W = _stream_waves(d)
        want = _al(batch * 2 * 2 * 4) + 2 * _al(2 * W * 4 * 4) + _al(2 * W * 4 * 128 * 4)
        assert pa.workspace_size(d) == want, (part, mbs, batch)
    # prefix folding (declared sharing, streaming path, G = 4 -> groups of 4):
    # the records of the groups' prefix streams after the sequences', state
    # rows of the 4 x 4 prefix columns per slot, the virtual lengths (5 per
    # group) and every stream's own state rows
    d = _desc(batch=8, path="mfma_stream", kv_shared=True)
    W, groups, rps = _stream_waves(d), 2, 16
    orows = (8 + groups) * 2 * rps
    want = (_al((8 + groups) * 2 * 2 * 4) + 2 * _al(2 * W * rps * 4) + _al(2 * W * rps * 128 * 4)
            + _al(groups * 5 * 4) + 2 * _al(orows * 4) + _al(orows * 128 * 4))
    assert pa.workspace_size(d) == want
    # no folding: one sequence, G = 16, or another kernel
    for kw in (dict(batch=1), dict(num_q_heads=32), dict(path="mfma_grid", partition_size=64)):
        args = dict(dict(batch=8, path="mfma_stream"), **kw)
        assert pa.workspace_size(_desc(kv_shared=True, **args)) == pa.workspace_size(_desc(**args)), kw
    # automatic choice: 4096 for the streaming kernel; for the others 512,
    # halved while the grid would be small
    assert pa.partition_size(_desc(batch=1, max_blocks_per_seq=6250, num_blocks=6250,
                                   path="mfma_stream")) == 4096
    assert pa.partition_size(_desc(max_blocks_per_seq=5120, num_blocks=16384)) == 4096
    auto = pa.partition_size(_desc(batch=1, max_blocks_per_seq=6250, num_blocks=6250, path="mfma_grid"))
    assert auto in (64, 128, 256, 512)
    big = pa.partition_size(_desc(batch=64, num_kv_heads=8, num_q_heads=64, path="mfma_grid",
                                  max_blocks_per_seq=2048, num_blocks=50000))
    assert big == 512
    # monotone in batch and in max_blocks_per_seq
    for path in ("mfma_grid", "auto"):
        sizes = [pa.workspace_size(_desc(batch=b, partition_size=32, path=path)) for b in (1, 2, 4, 8)]
        assert sizes == sorted(sizes) and sizes[0] > 0
        sizes = [pa.workspace_size(_desc(max_blocks_per_seq=m, partition_size=32, path=path))
                 for m in (4, 8, 16, 32)]
        assert sizes == sorted(sizes)


def test_check_inputs_on_host_copies():
    d = _desc(batch=3, max_blocks_per_seq=4, block_size=16, num_blocks=10)
    table = np.array([[0, 1, -1, -1], [2, -1, -1, -1], [3, 4, 5, 6]], dtype=np.int32)
    L = np.array([20, 16, 64], dtype=np.int32)
    assert pa.check_inputs(d, table, L) == 0
    t2 = table.copy(); t2[0, 1] = -1
    assert pa.check_inputs(d, t2, L) == -12           # -1 inside the attended range
    t2 = table.copy(); t2[2, 3] = 10
    assert pa.check_inputs(d, t2, L) == -12           # id >= num_blocks
    L2 = L.copy(); L2[2] = 65
    assert pa.check_inputs(d, table, L2) == -13       # beyond MBS * bs
    L2 = L.copy(); L2[1] = -1
    assert pa.check_inputs(d, table, L2) == -13
    L2 = L.copy(); L2[0] = 0
    assert pa.check_inputs(d, table, L2) == 0         # empty sequence reads nothing


def test_decode_argument_errors_return_before_device_work():
    d = _desc()
    good = 1 << 20  # never dereferenced: every call below fails validation first
    args = dict(q_ptr=good, k_ptr=good, v_ptr=good, table_ptr=good, seqlens_ptr=good, scale=1.0,
                out_ptr=good, ws_ptr=0, ws_bytes=0, status_ptr=0, stream=0)
    assert pa.decode_raw(_desc(head_dim=100), **args) == -3
    assert pa.decode_raw(d, **{**args, "q_ptr": 0}) == -1
    assert pa.decode_raw(d, **{**args, "out_ptr": good + 8}) == -7
    dw = _desc(partition_size=64)
    assert pa.workspace_size(dw) > 0
    assert pa.decode_raw(dw, **args) == -9                                   # no workspace
    assert pa.decode_raw(dw, **{**args, "ws_ptr": good, "ws_bytes": 16}) == -9  # too small
    assert pa.decode_raw(dw, **{**args, "ws_ptr": good + 16,
                                "ws_bytes": pa.workspace_size(dw)}) == -9    # misaligned
    assert pa.decode_raw(_desc(batch=0), **{**args, "q_ptr": 0}) == 0        # nothing to do


def _xp(**kw):
    # x-packed K [64, 2, 16, 16, 8] / V [64, 2, 128, 16]: block and head strides,
    # token strides x = 8 and 1
    base = dict(k_strides=(2 * 16 * 128, 16 * 128, 8), v_strides=(2 * 16 * 128, 16 * 128, 1),
                xpacked=True)
    base.update(kw)
    return _desc(**base)


def test_xpacked_layout_descriptor():
    assert pa.validate(_xp()) == 0
    # the grid kernels read it; AUTO and MFMA pick the grid kernel
    assert pa.PATH_NAME[pa.resolved_path(_xp())] == "mfma_grid"
    assert pa.PATH_NAME[pa.resolved_path(_xp(path="mfma"))] == "mfma_grid"
    assert pa.PATH_NAME[pa.resolved_path(_xp(path="mfma_fused"))] == "mfma_fused"
    assert pa.validate(_xp(path="mfma_stream")) == -10
    assert pa.validate(_xp(path="valu")) == -10
    assert pa.validate(_xp(kv_dtype="f32", k_strides=(4096, 2048, 4),
                           v_strides=(4096, 2048, 1))) == -10
    # token strides fixed by the layout; head stride holds the whole tile
    assert pa.validate(_xp(k_strides=(4096, 2048, 128))) == -6
    assert pa.validate(_xp(v_strides=(4096, 2048, 2))) == -6
    assert pa.validate(_xp(k_strides=(4096, 1024, 8))) == -6
    # a V^T piece is 8 tokens of one block
    assert pa.validate(_xp(block_size=4, k_strides=(2 * 4 * 128, 4 * 128, 8),
                           v_strides=(2 * 4 * 128, 4 * 128, 1))) == -4
    assert pa.validate(_xp(block_size=8, k_strides=(2 * 8 * 128, 8 * 128, 8),
                           v_strides=(2 * 8 * 128, 8 * 128, 1))) == 0


def test_flags_field():
    assert pa.validate(_desc(kv_shared=True)) == 0
    assert pa.validate(_desc(qo_bf16=True)) == 0
    assert pa.validate(_desc(kv_shared=True, qo_bf16=True)) == 0
    d = _desc()
    d.flags = 8  # unknown bit
    assert pa.validate(d) == -2
    d = _desc()
    d.reserved = 1
    assert pa.validate(d) == -2


def test_decode_append_argument_errors():
    d = _desc()
    good = 1 << 20  # never dereferenced: every call below fails before any launch
    args = dict(q_ptr=good, knew_ptr=good, vnew_ptr=good, k_ptr=good, v_ptr=good, table_ptr=good,
                seqlens_ptr=good, scale=1.0, out_ptr=good, ws_ptr=good,
                ws_bytes=pa.workspace_size(d), status_ptr=0, stream=0)
    assert pa.decode_append_raw(_desc(head_dim=100), **args) == -3
    assert pa.decode_append_raw(d, **{**args, "knew_ptr": 0}) == -1
    assert pa.decode_append_raw(d, **{**args, "vnew_ptr": 0}) == -1
    assert pa.decode_append_raw(d, **{**args, "vnew_ptr": good + 8}) == -7
    assert pa.decode_append_raw(_desc(batch=0), **{**args, "knew_ptr": 0}) == 0  # nothing to do


def test_prefill_argument_errors():
    """Every call below fails (or has nothing to do) before any launch."""
    d = _desc()
    good = 1 << 20
    args = dict(q_ptr=good, k_ptr=good, v_ptr=good, table_ptr=good, cu_q_ptr=good,
                seqlens_k_ptr=good, max_seqlen_q=16, causal=True, scale=1.0, out_ptr=good,
                ws_ptr=0, ws_bytes=0, status_ptr=0, stream=0)
    assert pa.prefill_raw(_desc(head_dim=100), **args) == -3              # bad descriptor
    assert pa.prefill_raw(d, **{**args, "cu_q_ptr": 0}) == -1            # no cu_seqlens_q
    assert pa.prefill_raw(d, **{**args, "seqlens_k_ptr": 0}) == -1       # no key lengths
    assert pa.prefill_raw(d, **{**args, "q_ptr": good + 4}) == -7        # misaligned
    assert pa.prefill_raw(_desc(kv_dtype="f32", k_strides=(4096, 2048, 128)), **args) == -10
    assert pa.prefill_raw(_xp(), **args) == -10   # x-packed caches: decode only
    assert pa.prefill_raw(_desc(block_size=8, k_strides=(2048, 1024, 128)), **args) == -2
    assert pa.prefill_raw(d, **{**args, "max_seqlen_q": -1}) == -2
    assert pa.prefill_raw(d, **{**args, "max_seqlen_q": 0}) == 0          # no rows
    assert pa.prefill_raw(_desc(batch=0), **{**args, "cu_q_ptr": 0}) == 0  # no sequences
    # no workspace is involved, whatever the decode would need
    assert pa.workspace_size(d) > 0
    assert pa.prefill_workspace_size(d, 16) == 0
    # a launch that splits keys: a workspace smaller than its size, or not
    # 256-byte aligned, is refused
    p1 = _desc(batch=4, num_q_heads=24, num_kv_heads=4, head_dim=256, max_blocks_per_seq=512,
               num_blocks=2048, k_strides=(4 * 16 * 256, 16 * 256, 256))
    n = pa.prefill_workspace_size(p1, 512)
    assert n > 0
    a1 = {**args, "max_seqlen_q": 512}
    assert pa.prefill_raw(p1, **{**a1, "ws_ptr": good, "ws_bytes": n - 1}) == -9
    assert pa.prefill_raw(p1, **{**a1, "ws_ptr": good + 16, "ws_bytes": n}) == -7


def test_prefill_key_split_workspace():
    """The key split's plan, for 256 compute units (the host's count when no GPU
    is visible) and 8 XCDs. Work items per XCD: the (sequence, KV head) pairs
    dealt round robin (ceil(B Hkv / 8) rounds of pairs) times the items per pair
    (16-row tile groups x head groups); the workgroups an XCD holds at once: 32
    compute units x (1 at d = 256; at d = 128 3 with bf16 q over bf16 K/V, else
    2). A last round at most half full is split: counters (8 x split items
    int32, 256-byte aligned) then two halves' states (8 units x (d/16 x 256 +
    128) floats) per split item."""
    def desc(B, Hq, Hkv, D, bf=True, kv="bf16"):
        return _desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, max_blocks_per_seq=512,
                     num_blocks=2048, k_strides=(Hkv * 16 * D, 16 * D, D), qo_bf16=bf, kv_dtype=kv)
    def want(nsplit, D):
        cnt = (8 * nsplit * 4 + 255) // 256 * 256
        return cnt + 8 * nsplit * 2 * 8 * ((D // 16) * 256 + 128) * 4, 8 * nsplit * 4
    # d = 256, G = 6 (two heads x four tiles per workgroup): 512 rows -> 24 items
    # per pair; 16 pairs -> 2 rounds of pairs -> 48 items per XCD = 32 + 16:
    # the 16 are split (fp32 and bf16 q/out alike)
    for bf in (True, False):
        d = desc(4, 24, 4, 256, bf)
        assert (pa.prefill_workspace_size(d, 512), pa.prefill_workspace_zeroed_bytes(d, 512)) == want(16, 256)
    # 256 rows -> 12 items per pair, 8 pairs -> 12 items per XCD: fewer than 32
    assert pa.prefill_workspace_size(desc(2, 24, 4, 256), 256) == 0
    # 24 pairs -> 72 items per XCD = 2 x 32 + 8: the 8 are split; 32 pairs ->
    # 96 = 3 x 32: none
    assert pa.prefill_workspace_size(desc(6, 24, 4, 256), 512) == want(8, 256)[0]
    assert pa.prefill_workspace_size(desc(8, 24, 4, 256), 512) == 0
    # d = 128, G = 8 (eight heads x one tile): 256 rows -> 16 items per pair.
    # bf16 q over bf16 K/V (96 per XCD at once): 128 pairs -> 256 items = 2 x 96
    # + 64: more than half, none; 112 pairs -> 224 = 2 x 96 + 32: 32 split;
    # 40 pairs -> 80: fewer than 96
    assert pa.prefill_workspace_size(desc(16, 64, 8, 128), 256) == 0
    assert pa.prefill_workspace_size(desc(14, 64, 8, 128), 256) == want(32, 128)[0]
    assert pa.prefill_workspace_size(desc(5, 64, 8, 128), 256) == 0
    # fp32 q, or bf16 q over fp16 K/V (64 per XCD at once): 40 pairs -> 80 =
    # 64 + 16: 16 split
    assert pa.prefill_workspace_size(desc(5, 64, 8, 128, bf=False), 256) == want(16, 128)[0]
    assert pa.prefill_workspace_size(desc(5, 64, 8, 128, kv="f16"), 256) == want(16, 128)[0]
    # refused descriptors and no rows: 0
    assert pa.prefill_workspace_size(desc(4, 24, 4, 256), 0) == 0
    assert pa.prefill_workspace_size(_desc(kv_dtype="f32", k_strides=(4096, 2048, 128)), 512) == 0


def test_decode_static_refuses_before_device_work():
    """The allocation-free decode checks the descriptor, the path and the
    workspace it would need against its static scratch before it touches any
    device: too large a need returns PA_E_SCRATCH, the merged grid variant
    PA_E_PATH (its arrival counters would have to be zero in the shared
    array), a bad descriptor its own code; nothing runs, so null pointers are
    never looked at."""
    lib = pa.load_library()
    assert pa.PA_STATIC_SCRATCH_BYTES == 32 << 20

    def call(d):
        return _lib.decode_static_raw(d, 0, 0, 0, 0, 0, 1.0, 0, 0, 0)

    # the 64-sequence batch on the grid kernel at 512-token partitions: ~130 MiB
    big = pa.make_desc(batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                       num_blocks=45000, max_blocks_per_seq=2048, kv_dtype="bf16",
                       k_strides=(8 * 16 * 128, 16 * 128, 128), partition_size=512,
                       path="mfma_grid")
    assert pa.workspace_size(big) > pa.PA_STATIC_SCRATCH_BYTES
    assert call(big) == -16
    assert lib.paged_attn_strerror(-16).decode().startswith("the call needs more workspace")
    fused = pa.make_desc(batch=4, num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                         num_blocks=100, max_blocks_per_seq=64, kv_dtype="bf16",
                         k_strides=(2 * 16 * 128, 16 * 128, 128), partition_size=64,
                         path="mfma_fused")
    assert call(fused) == -10
    bad = pa.make_desc(batch=4, num_q_heads=16, num_kv_heads=2, head_dim=96, block_size=16,
                       num_blocks=100, max_blocks_per_seq=64, kv_dtype="bf16",
                       k_strides=(2 * 16 * 96, 16 * 96, 96))
    assert call(bad) == -3
