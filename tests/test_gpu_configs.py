"""GPU parity on the five decode workloads at full size: the WHOLE output of
every kernel path against the fp64 oracle, element by element.

Each workload is drawn once (``util_cases.config_case``) and the oracle runs
once over every (sequence, query head) of it; then each variant below runs the
same batch through the C ABI and is compared in full. Tolerance (max-abs): 1e-5
for fp32 K/V, 3e-3 for fp16/bf16 K/V. Every slot no sequence attends to holds
NaN, so any read of one would show as a non-finite output.

Variants:
  bench        exactly the launch ``bench.py`` times: its ``Workload`` object,
               library-chosen path and partition size (512 fixed for the
               100K-token workload), cacheable K/V loads for the prefix-shared
               workload, non-temporal loads otherwise
  stream/grid/valu/fused
               each partition kernel forced, at the library's partition size
               or a fixed one (so partition counts other than the default are
               covered too)
  xpacked      the x-packed K / transposed V pools (same values)
  shared       the prefix-shared workload on the streaming kernel without the
               shared-blocks flag, and the automatic path with it
"""
import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from paged_gqa_decode_block_amd import workload as W
from util_cases import config_case, config_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3, "bf16": 3e-3}

# (variant, path, partition size, kv_shared); partition None = the workload's own
VARIANTS = {
    1: [("bench", None, None, None), ("valu", "valu", 0, False), ("valu", "valu", 32, False)],
    2: [("bench", None, None, None), ("stream", "mfma_stream", 0, False),
        ("stream", "mfma_stream", 64, False), ("grid", "mfma_grid", 0, False),
        ("valu", "valu", 0, False), ("fused", "mfma_fused", 0, False),
        ("xpacked", "mfma_grid", 0, False)],
    3: [("bench", None, None, None), ("stream", "mfma_stream", 0, False),
        ("grid", "mfma_grid", 512, False), ("valu", "valu", 512, False),
        ("fused", "mfma_fused", 0, False), ("xpacked", "mfma_grid", 512, False)],
    4: [("bench", None, None, None), ("stream", "mfma_stream", 512, False),
        ("grid", "mfma_grid", 0, False), ("valu", "valu", 0, False),
        ("fused", "mfma_fused", 0, False), ("xpacked", "mfma_grid", 0, False)],
    5: [("bench", None, None, None), ("shared", "mfma_stream", 0, False),
        ("shared", "auto", 512, True), ("grid", "mfma_grid", 0, False),
        ("valu", "valu", 0, False), ("fused", "mfma_fused", 0, False),
        ("xpacked", "mfma_grid", 0, False)],
}
PARAMS = [(k, i) for k in sorted(VARIANTS) for i in range(len(VARIANTS[k]))]

_DEV = {}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()  # fail loudly if the HIP library is missing
    return torch


def _device(torch, case, k, layout):
    """The workload's tensors on the GPU (guard block dropped), cached for
    workload k in one layout at a time."""
    key = (k, layout)
    if key in _DEV:
        return _DEV[key]
    _DEV.clear()
    torch.cuda.empty_cache()

    def pool(store, which):
        if case.kv_dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(store)).to("cuda")[1:]
        if layout == "XPACKED":
            store = W.to_xpacked(store, which)
        t = torch.from_numpy(np.ascontiguousarray(store).view(np.int16))
        return t.view(torch.bfloat16 if case.kv_dtype == "bf16" else torch.float16).to("cuda")[1:]

    _DEV[key] = dict(q=torch.from_numpy(case.q).to("cuda"), k=pool(case.k_store, "k"),
                     v=pool(case.v_store, "v"),
                     table=torch.from_numpy(case.block_table).to("cuda"),
                     seqlens=torch.from_numpy(case.seqlens).to("cuda"))
    return _DEV[key]


@pytest.mark.parametrize("k,i", PARAMS,
                         ids=[f"c{k}-{VARIANTS[k][i][0]}-{VARIANTS[k][i][1] or 'bench'}-"
                              f"{VARIANTS[k][i][2]}" for k, i in PARAMS])
def test_workload_whole_output_matches_oracle(torch_cuda, k, i):
    torch = torch_cuda
    variant, path, part, shared = VARIANTS[k][i]
    case = config_case(k)
    want = config_oracle(k)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if variant == "bench":
        import bench

        _DEV.clear()
        wl = bench.Workload(k, torch, "auto", case=case)
        wl.call()
        torch.cuda.synchronize()
        got = wl.out.cpu().numpy().astype(np.float64)
        print(f"c{k} bench launch: path {wl.path_name}, partition {wl.part}, "
              f"kv_shared {wl.kv_shared}")
        del wl
        torch.cuda.empty_cache()
    else:
        layout = "XPACKED" if variant == "xpacked" else case.layout
        dev = _device(torch, case, k, layout)
        got = pa.paged_attn_decode(dev["q"], dev["k"], dev["v"], dev["table"], dev["seqlens"],
                                   case.scale, layout=layout, partition_size=part, path=path,
                                   status=status, kv_shared=shared)
        torch.cuda.synchronize()
        got = got.cpu().numpy().astype(np.float64)
        assert int(status.item()) == 0, (k, variant, path, part)
    assert got.shape == want.shape
    assert np.isfinite(got).all(), (k, variant, path, part)
    err = float(np.abs(got - want).max())
    print(f"c{k} {variant} {path} partition {part}: max-abs error {err:.3e} over {got.size} values")
    assert err <= TOL[case.kv_dtype], (k, variant, path, part, err)
