"""GPU: paged_attn_decode_static, the decode that allocates nothing (its partial
states live in the library's static scratch array), against paged_attn_decode
with a caller workspace, through the C ABI.

Two calls in a row on each kernel path, the second with a smaller batch (fewer
sequences, fewer heads, shorter contexts), so the second runs over the first
call's leftovers in the shared array. Each output must equal the workspace
call's bit for bit (same kernels, same partition size, same workspace layout)
and lie within the K/V tolerance of the fp64 oracle. Also: a captured HIP graph
of the static call replays equal to eager calls, and a call needing more than
the static array is refused before any launch.
"""
import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from util_cases import paged_case, run_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3, "bf16": 3e-3}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()
    return torch


def _device(torch, case):
    def pool(store):
        if case.kv_dtype == "f32":
            t = torch.from_numpy(np.ascontiguousarray(store))
        else:
            t = torch.from_numpy(np.ascontiguousarray(store).view(np.int16))
            t = t.view(torch.bfloat16 if case.kv_dtype == "bf16" else torch.float16)
        return t.to("cuda")[1:]

    return (torch.from_numpy(case.q).to("cuda"), pool(case.k_store), pool(case.v_store),
            torch.from_numpy(case.block_table).to("cuda"),
            torch.from_numpy(case.seqlens).to("cuda"))


# path, head_dim, KV dtype, partition size, (B, Hq, Hkv, lengths) of the first and second call
CASES = [
    ("mfma_stream", 128, "bf16", 0, (6, 32, 4, [3000, 17, 1500, 0, 700, 2222]), (3, 16, 2, [900, 33, 1])),
    ("mfma_stream", 256, "bf16", 512, (2, 24, 4, [5000, 1200]), (1, 12, 2, [700])),
    ("mfma_grid", 128, "f16", 64, (5, 16, 2, [1000, 64, 2049, 5, 300]), (2, 8, 2, [129, 40])),
    ("valu", 64, "f32", 32, (4, 8, 2, [500, 31, 0, 260]), (2, 4, 2, [70, 1])),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[f"{c[0]}-d{c[1]}-{c[2]}" for c in CASES])
def test_static_equals_workspace_call_two_calls_in_a_row(torch_cuda, idx):
    torch = torch_cuda
    path, D, dt, part, first, second = CASES[idx]
    rng = np.random.default_rng(3000 + idx)
    for step, (B, Hq, Hkv, L) in enumerate((first, second)):
        case, _, _ = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=16, kv_dtype=dt, seqlens=L,
                                spare=3)
        q, k, v, table, seqlens = _device(torch, case)
        kw = dict(partition_size=part, path=path)
        ref = pa.paged_attn_decode(q, k, v, table, seqlens, case.scale, **kw)
        out = torch.full_like(q, float("nan"))
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        print(f"static decode: {path} d={D} {dt} call {step + 1}, B={B}", flush=True)
        pa.paged_attn_decode_static(q, k, v, table, seqlens, case.scale, out, status=status, **kw)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, (path, step)
        assert torch.equal(out, ref), (path, step)
        got = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), (path, step)
        assert np.abs(got - run_oracle(case)).max() <= TOL[dt], (path, step)


def test_static_call_graph_replay(torch_cuda):
    """The static call captured once in a HIP graph (nothing to allocate, so it
    captures as is) and replayed with new q values copied in between: every
    replay equals an eager static call bit for bit."""
    torch = torch_cuda
    rng = np.random.default_rng(3100)
    case, _, _ = paged_case(rng, B=4, Hq=16, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[2500, 33, 900, 1])
    q, k, v, table, seqlens = _device(torch, case)
    q_s = q.clone()
    out_s = torch.zeros_like(q)
    kw = dict(partition_size=0, path="mfma_stream")
    pa.paged_attn_decode_static(q_s, k, v, table, seqlens, case.scale, out_s, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.paged_attn_decode_static(q_s, k, v, table, seqlens, case.scale, out_s, **kw)
    torch.cuda.synchronize()
    for step in range(3):
        if step:
            q_s.copy_(torch.randn_like(q_s))
        g.replay()
        torch.cuda.synchronize()
        got = out_s.clone()
        eager = torch.empty_like(q_s)
        pa.paged_attn_decode_static(q_s, k, v, table, seqlens, case.scale, eager, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), step
        if step == 0:
            assert np.abs(got.cpu().numpy().astype(np.float64) - run_oracle(case)).max() <= 3e-3


def test_static_call_refuses_a_workspace_beyond_the_array(torch_cuda):
    """A descriptor whose workspace exceeds PA_STATIC_SCRATCH_BYTES returns
    PA_E_SCRATCH and leaves the output untouched."""
    torch = torch_cuda
    rng = np.random.default_rng(3200)
    case, _, _ = paged_case(rng, B=2, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="bf16", seqlens=[40, 9])
    q, k, v, table, seqlens = _device(torch, case)
    # a table 2^16 blocks wide at 32-token partitions: 2 x 8 heads x 32768
    # partitions of states, about 270 MB, far beyond the 32 MiB array
    wide = torch.full((2, 1 << 16), -1, dtype=torch.int32, device="cuda")
    wide[:, : table.shape[1]] = table
    out = torch.full_like(q, 7.0)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_attn_decode_static(q, k, v, wide, seqlens, case.scale, out, partition_size=32,
                                    path="mfma_grid")
    assert e.value.code == -16
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
