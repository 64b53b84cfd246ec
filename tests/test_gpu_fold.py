"""GPU parity of prefix folding on the streaming path: sequences that declare
shared blocks (kv_shared) are grouped F = 16 / G at a time, and the leading
blocks a group's members all list and attend whole are read once, with the
F x G query heads in the score MFMA's columns. Every output is compared with
the fp64 oracle (which knows nothing of the sharing): groups that fold, groups
that do not (members of different families, a member shorter than the
minimum prefix), a member whose length ends exactly at the prefix (nothing of
its own), a prefix cut short by one member's private copy of a block, G = 2,
4, 6, 8 and 16 (no folding), head sizes 64, 128, 256, both layouts, fp16 and
bf16."""
import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from util_cases import run_oracle, shared_prefix_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()
    return torch


CASES = [
    # name, Hq, Hkv, D, bs, dtype, layout, families, mismatch, folds
    ("g4_d128", 16, 4, 128, 16, "bf16", "HND",
     [(40, [700, 640, 900, 641]), (36, [576, 600, 700, 1100, 590]), (20, [330, 100, 500])],
     None, True),
    ("g4_d128_cut", 16, 4, 128, 16, "bf16", "HND",
     [(40, [700, 660, 900, 680]), (24, [500, 400, 384, 450])], (0, 2, 20), True),
    ("g8_d128_bs32_nhd", 32, 4, 128, 32, "f16", "NHD",
     [(24, [800, 768]), (10, [400, 330]), (30, [1000, 961, 1200])], None, True),
    ("g2_d64", 8, 4, 64, 16, "bf16", "HND",
     [(32, [600, 512, 530, 700, 900, 513, 520, 1000]), (20, [400, 330])], None, True),
    ("g4_d256", 16, 4, 256, 16, "bf16", "HND",
     [(32, [600, 512, 530, 700]), (16, [300, 280, 257, 400])], None, True),
    ("g6_d128", 12, 2, 128, 16, "bf16", "HND",
     [(30, [500, 480]), (30, [700, 481]), (8, [200, 150])], None, True),
    ("g16_d128", 32, 2, 128, 16, "bf16", "HND",
     [(30, [500, 480, 600])], None, False),
]


def _device(torch, case):
    def pool(store):
        t = torch.from_numpy(np.ascontiguousarray(store).view(np.int16))
        return t.view(torch.bfloat16 if case.kv_dtype == "bf16" else torch.float16).to("cuda")[1:]

    return (torch.from_numpy(case.q).to("cuda"), pool(case.k_store), pool(case.v_store),
            torch.from_numpy(case.block_table).to("cuda"), torch.from_numpy(case.seqlens).to("cuda"))


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_fold_matches_oracle(torch_cuda, idx):
    torch = torch_cuda
    name, Hq, Hkv, D, bs, dt, layout, fams, mismatch, folds = CASES[idx]
    rng = np.random.default_rng(1500 + idx)
    case = shared_prefix_case(rng, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=dt, families=fams,
                              layout=layout, mismatch=mismatch)
    q, k, v, table, seqlens = _device(torch, case)
    # folding is on exactly when the declared sharing gives it a group layout
    shared = pa.desc_for(q, k, v, table, layout=layout, path="mfma_stream", kv_shared=True)
    plain = pa.desc_for(q, k, v, table, layout=layout, path="mfma_stream")
    assert (pa.workspace_size(shared) > pa.workspace_size(plain)) == folds
    want = run_oracle(case)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rep in range(2):  # the second call reuses the workspace the first left
        out = pa.paged_attn_decode(q, k, v, table, seqlens, case.scale, layout=layout,
                                   path="mfma_stream", status=status, kv_shared=True)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert int(status.item()) == 0
        assert np.isfinite(got).all()
        err = np.abs(got - want).max()
        assert err <= 3e-3, (name, rep, err)
