"""GPU parity of the x-packed K / transposed V cache layout (PA_FLAG_KV_XPACKED:
K [NB, H_kv, d/8, bs, 8], V [NB, H_kv, d, bs], the layout of page "Paged
Attention Kernel Architecture for BI-V100", section 3).

Each case is drawn in the default [NB, H_kv, bs, d] layout (NaN guard block and
NaN poison in every unattended slot) and handed to the GPU permuted into the
x-packed layout (workload.to_xpacked, pinned on the CPU), while the oracle reads
the unpermuted pool. Lengths that are not multiples of 8 put the sequence end
inside a V^T piece: a read of the poisoned slots after it would turn the output
NaN. The grid kernel reads the same K fragments and the same V values in the
same order in both layouts, so its output must not change by a bit.
"""
import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from paged_gqa_decode_block_amd import workload as W
from test_gpu_parity import (  # noqa: F401  (torch_cuda is a fixture)
    TOL, _append_case, _append_host, _new_token, run_gpu, to_device, torch_cuda)
from util_cases import paged_case, run_oracle

pytestmark = pytest.mark.gpu


def to_device_xp(torch, case):
    """The case's pools on the device in the x-packed layout (guard block dropped)."""
    assert case.layout == "HND" and case.kv_dtype in ("f16", "bf16")
    tdt = torch.bfloat16 if case.kv_dtype == "bf16" else torch.float16

    def pool(store, which):
        a = W.to_xpacked(store, which)
        return torch.from_numpy(a.view(np.int16)).view(tdt).to("cuda")[1:]

    dev = to_device(torch, case)
    dev["k"] = pool(case.k_store, "k")
    dev["v"] = pool(case.v_store, "v")
    return dev


def run_xp(torch, case, dev, *, path="auto", partition_size=0):
    out = pa.paged_attn_decode(dev["q"], dev["k"], dev["v"], dev["table"], dev["seqlens"],
                               case.scale, layout="XPACKED", partition_size=partition_size,
                               path=path)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


XP_CASES = [
    # name, B, Hq, Hkv, D, bs, dtype, seqlens, partition
    ("bf16_d128_g8_bs16", 4, 32, 4, 128, 16, "bf16", [31, 32, 33, 700], 64),
    ("f16_d64_g7_bs8", 3, 14, 2, 64, 8, "f16", [513, 1, 100], 32),
    ("bf16_d256_g6_bs16", 1, 24, 4, 256, 16, "bf16", [1003], 512),
    ("bf16_d128_g4_bs32", 3, 16, 4, 128, 32, "bf16", [2049, 5, 64], 512),
    ("f16_d128_g1_bs64", 2, 4, 4, 128, 64, "f16", [300, 63], 96),
    ("bf16_d256_g16_bs8", 2, 32, 2, 256, 8, "bf16", [77, 250], 32),
    ("bf16_empty_and_one", 4, 8, 2, 128, 16, "bf16", [0, 1, 0, 17], 32),
]


@pytest.mark.parametrize("idx", range(len(XP_CASES)), ids=[c[0] for c in XP_CASES])
def test_xpacked_small_cases(torch_cuda, idx):
    torch = torch_cuda
    name, B, Hq, Hkv, D, bs, dt, L, part = XP_CASES[idx]
    rng = np.random.default_rng(700 + idx)
    case, _, _ = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=dt, seqlens=L, spare=4)
    want = run_oracle(case)
    dev_hnd = to_device(torch, case)
    dev = to_device_xp(torch, case)
    for path in ("mfma_grid", "mfma_fused", "auto"):
        for ps in (part, 0):
            got = run_xp(torch, case, dev, path=path, partition_size=ps)
            assert np.isfinite(got).all(), (name, path, ps)
            err = np.abs(got - want).max()
            assert err <= TOL[dt], (name, path, ps, err)
            # the default layout on the same kernel gives the same bits
            ref = run_gpu(torch, case, dev_hnd, path="mfma_grid" if path == "auto" else path,
                          partition_size=ps)
            assert np.array_equal(got, ref), (name, path, ps)


def test_xpacked_append(torch_cuda):
    """Two decode steps that append the new token in place into x-packed caches:
    each matches the oracle on the updated cache, and the device pools then equal
    the permuted host pools bit for bit (the future slots hold NaN until
    written)."""
    torch = torch_cuda
    rng = np.random.default_rng(130)
    case = _append_case(rng, kv_dtype="bf16", L0=(100, 31, 200), D=128, bs=16)
    dev = to_device_xp(torch, case)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for step in range(2):
        q, kn, vn, qd, knd, vnd = _new_token(torch, rng, case)
        out = pa.paged_attn_decode_append(qd, knd, vnd, dev["k"], dev["v"], dev["table"],
                                          dev["seqlens"], case.scale, layout="XPACKED",
                                          partition_size=32, status=status)
        torch.cuda.synchronize()
        case = _append_host(case, q, kn, vn)
        got = out.cpu().numpy().astype(np.float64)
        assert np.abs(got - run_oracle(case)).max() <= 3e-3, step
        for which, t in (("k", dev["k"]), ("v", dev["v"])):
            host = W.to_xpacked(case.k_store if which == "k" else case.v_store, which)[1:]
            assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), host), (step, which)
        dev["seqlens"] += 1
    assert int(status.item()) == 0


def test_xpacked_copy_blocks(torch_cuda):
    """Whole-block device copies in x-packed pools equal the same copies of the
    permuted host pools."""
    torch = torch_cuda
    rng = np.random.default_rng(131)
    case, _, _ = paged_case(rng, B=2, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[100, 50], spare=4)
    dev = to_device_xp(torch, case)
    NB = case.NB
    pairs = np.array([[0, NB - 1], [3, NB - 2]], dtype=np.int32)
    pa.copy_blocks(dev["k"], dev["v"], torch.from_numpy(pairs).to("cuda"), layout="XPACKED")
    torch.cuda.synchronize()
    for which, t, store in (("k", dev["k"], case.k_store), ("v", dev["v"], case.v_store)):
        host = W.to_xpacked(store, which)[1:].copy()
        for s, d in pairs:
            host[d] = host[s]
        assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), host), which
