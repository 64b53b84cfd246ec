"""GPU parity of the merged-grid path (PA_PATH_MFMA_FUSED): the grid MFMA kernel
whose last partition workgroup of each (sequence, KV head) merges the partition
states in the same launch, through arrival counters at the start of the
workspace.

Against the fp64 oracle at the K/V tolerance (3e-3) on the small cases at
several partition sizes (many partitions per sequence), across back-to-back calls whose partition
counts differ (the counters must come back to zero after every call), under
graph replay, and with bad table entries. Every call goes through the C ABI.
"""
import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from paged_gqa_decode_block_amd import workload as W
from test_gpu_parity import (  # noqa: F401  (torch_cuda is a fixture)
    SMALL, TOL, run_gpu, to_device, torch_cuda)
from util_cases import paged_case, run_oracle

pytestmark = pytest.mark.gpu

FUSED = "mfma_fused"
SMALL16 = [i for i, s in enumerate(SMALL) if s[6] != "f32"]


@pytest.mark.parametrize("idx", SMALL16, ids=[SMALL[i][0] for i in SMALL16])
def test_small_cases_fused(torch_cuda, idx):
    name, B, Hq, Hkv, D, bs, dt, layout, L, part = SMALL[idx]
    rng = np.random.default_rng(500 + idx)
    case, _, _ = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=dt, seqlens=L,
                            layout=layout, spare=4)
    want = run_oracle(case)
    dev = to_device(torch_cuda, case)
    ran = 0
    for ps in (part, 32, 0):
        try:
            got = run_gpu(torch_cuda, case, dev, path=FUSED, partition_size=ps)
        except pa.PagedAttnError as e:
            assert e.code == -8, (name, ps, e)  # only the merge's LDS bound may refuse
            continue
        ran += 1
        assert np.isfinite(got).all(), (name, ps)
        err = np.abs(got - want).max()
        assert err <= TOL[dt], (name, ps, err)
    assert ran


def test_back_to_back_calls_leave_counters_zero(torch_cuda):
    """Three calls on one caller-owned workspace: lengths A, then shorter lengths
    B (other partition counts per sequence), then A again. Each matches the
    oracle, the third equals the first bit for bit, and after every call the
    arrival counters are zero again."""
    torch = torch_cuda
    rng = np.random.default_rng(120)
    case_a, _, _ = paged_case(rng, B=5, Hq=16, Hkv=4, D=128, bs=16, kv_dtype="bf16",
                              seqlens=[1500, 40, 700, 0, 3000])
    case_b = W.Case(**{**case_a.__dict__,
                       "seqlens": np.array([300, 17, 650, 0, 1111], dtype=np.int32)})
    dev = to_device(torch, case_a)
    ws = torch.zeros(32 << 20, dtype=torch.uint8, device="cuda")
    ncnt = case_a.B * case_a.Hkv

    def call(case):
        out = pa.paged_attn_decode(dev["q"], dev["k"], dev["v"], dev["table"],
                                   torch.from_numpy(case.seqlens).to("cuda"), case.scale,
                                   layout=case.layout, partition_size=32, path=FUSED, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[: 4 * ncnt].view(torch.int32).abs().sum().item()) == 0
        return out.cpu().numpy().astype(np.float64)

    want_a, want_b = run_oracle(case_a), run_oracle(case_b)
    a1 = call(case_a)
    assert np.abs(a1 - want_a).max() <= 3e-3
    b1 = call(case_b)
    assert np.abs(b1 - want_b).max() <= 3e-3
    a2 = call(case_a)
    assert np.array_equal(a1, a2)


def test_fused_matches_two_launch_grid(torch_cuda):
    """The merged variant and the two-launch grid path fold the same partition
    states; they differ only in the order of the merge's additions."""
    rng = np.random.default_rng(122)
    case, _, _ = paged_case(rng, B=3, Hq=24, Hkv=4, D=256, bs=16, kv_dtype="bf16",
                            seqlens=[5000, 512, 513])
    dev = to_device(torch_cuda, case)
    a = run_gpu(torch_cuda, case, dev, path=FUSED, partition_size=64)
    b = run_gpu(torch_cuda, case, dev, path="mfma_grid", partition_size=64)
    assert np.abs(a - b).max() <= 1e-5


def test_fused_graph_replay(torch_cuda):
    """The one-launch decode captured in a HIP graph and replayed with new q
    values copied in between: every replay equals an eager call bit for bit,
    and the first matches the oracle."""
    torch = torch_cuda
    rng = np.random.default_rng(121)
    case, _, _ = paged_case(rng, B=4, Hq=16, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[900, 33, 2000, 1])
    dev = to_device(torch, case)
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    q_s = dev["q"].clone()
    out_s = torch.zeros_like(q_s)
    args = (dev["k"], dev["v"], dev["table"], dev["seqlens"], case.scale)
    kw = dict(layout=case.layout, partition_size=64, path=FUSED)
    pa.paged_attn_decode(q_s, *args, out_s, workspace=ws, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.paged_attn_decode(q_s, *args, out_s, workspace=ws, **kw)
    torch.cuda.synchronize()
    want = run_oracle(case)
    for step in range(4):
        if step:
            q_s.copy_(torch.randn_like(q_s))
        g.replay()
        torch.cuda.synchronize()
        got = out_s.clone()
        eager = pa.paged_attn_decode(q_s, *args, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), step
        if step == 0:
            assert np.abs(got.cpu().numpy().astype(np.float64) - want).max() <= 3e-3


def test_fused_bad_entries_skipped_and_reported(torch_cuda):
    """An unassigned (-1) and an out-of-pool entry inside the attended range are
    never dereferenced (a read of the NaN guard or poison would make the output
    non-finite) and are reported in the status word; with the table repaired
    the same call reports nothing and matches the oracle."""
    torch = torch_cuda
    rng = np.random.default_rng(123)
    case, _, _ = paged_case(rng, B=3, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[700, 40, 20])
    good = case.block_table.copy()
    case.block_table[0, 3] = -1
    case.block_table[1, 0] = case.NB
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_gpu(torch, case, path=FUSED, partition_size=32, status=status)
    assert int(status.item()) & pa.PA_STATUS_BAD_BLOCK
    assert np.isfinite(got).all()
    case.block_table[:] = good
    status.zero_()
    got = run_gpu(torch, case, path=FUSED, partition_size=32, status=status)
    assert int(status.item()) == 0
    assert np.abs(got - run_oracle(case)).max() <= 3e-3
