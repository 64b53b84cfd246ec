"""GPU parity of the paged varlen prefill (paged_attn_prefill) against the
fp64 oracle, element by element: head sizes 64/128/256, fp16 and bf16 K/V,
HND and NHD pools, causal and full attention, sequences whose query count is
below, equal to and above their key count, empty sequences and rows with no
key to attend (zeros), several 16-row tiles with a ragged last one, bf16 q and
out, the status report for a max_seqlen_q below a sequence's row count, and
the key split of a last round of work items (halves merged in the kernel)."""
from __future__ import annotations

import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from oracle import oracle as O
from util_cases import paged_case

pytestmark = pytest.mark.gpu
TOL = {"f16": 3e-3, "bf16": 3e-3}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()
    return torch


def _pool(torch, case, store):
    t = torch.from_numpy(np.ascontiguousarray(store).view(np.int16))
    return t.view(torch.bfloat16 if case.kv_dtype == "bf16" else torch.float16).to("cuda")[1:]


def _make(rng, *, Hq, Hkv, D, bs, kv_dtype, klens, qlens, layout="HND", **kw):
    klens = np.asarray(klens, dtype=np.int32)
    qlens = np.asarray(qlens, dtype=np.int32)
    case, _, _ = paged_case(rng, B=len(klens), Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=kv_dtype,
                            seqlens=klens, layout=layout, **kw)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), Hq, D)).astype(np.float32)
    return case, cu, q


def _oracle(case, cu, q, causal):
    return O.paged_attn_prefill(q, case.k_pool, case.v_pool, case.block_table, cu, case.seqlens,
                                case.scale, causal=causal, kv_dtype=case.kv_dtype,
                                block_size=case.bs, num_kv_heads=case.Hkv, layout=case.layout)


def _gpu(torch, case, cu, q, causal, *, max_q=None, status=None, bf16=False, split=True):
    qd = torch.from_numpy(q).to("cuda")
    if bf16:
        qd = qd.to(torch.bfloat16)
    out = pa.paged_attn_prefill(qd, _pool(torch, case, case.k_store), _pool(torch, case, case.v_store),
                                torch.from_numpy(case.block_table).to("cuda"),
                                torch.from_numpy(cu).to("cuda"),
                                torch.from_numpy(case.seqlens).to("cuda"), case.scale,
                                max_seqlen_q=max_q, causal=causal, layout=case.layout, status=status,
                                split=split)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


CASES = [
    # name, Hq, Hkv, D, bs, dtype, layout, key lengths, query lengths
    ("d128_g8_mixed", 16, 2, 128, 16, "bf16", "HND", [300, 40, 77, 1], [37, 40, 90, 1]),
    ("d64_g7_f16", 14, 2, 64, 16, "f16", "HND", [513, 16, 0, 100], [16, 17, 5, 0]),
    ("d256_g6", 12, 2, 256, 16, "bf16", "HND", [700, 33], [65, 33]),
    ("d128_nhd_bs32", 8, 1, 128, 32, "bf16", "NHD", [250, 64], [31, 64]),
    ("d128_g1", 4, 4, 128, 64, "f16", "HND", [129, 200], [129, 3]),
    # G = 12: four heads times two tiles per workgroup; G = 2 at d = 64: two
    # units per wave on different tiles
    ("d128_g12", 24, 2, 128, 16, "bf16", "HND", [400, 90], [70, 90]),
    ("d64_g2_tiles", 8, 4, 64, 16, "bf16", "HND", [1000, 20], [200, 20]),
    # the largest group and the largest block: two 8-head units' groups, a
    # whole sequence inside one 1024-token block
    ("d128_g16_bs1024", 32, 2, 128, 1024, "bf16", "HND", [1500, 300], [70, 300]),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(torch_cuda, idx, causal):
    name, Hq, Hkv, D, bs, dt, layout, kl, ql = CASES[idx]
    rng = np.random.default_rng(1200 + idx)
    case, cu, q = _make(rng, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=dt, klens=kl, qlens=ql,
                        layout=layout)
    want = _oracle(case, cu, q, causal)
    status = torch_cuda.zeros(1, dtype=torch_cuda.int32, device="cuda")
    got = _gpu(torch_cuda, case, cu, q, causal, status=status)
    assert int(status.item()) == 0
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= TOL[dt], (name, causal, err)
    # rows that attend nothing are exact zeros
    for b in range(len(kl)):
        for i in range(ql[b]):
            if causal and kl[b] - ql[b] + i + 1 <= 0 or kl[b] == 0:
                assert np.all(got[cu[b] + i] == 0.0)


def test_prefill_last_row_is_the_decode(torch_cuda):
    """The last causal row of every sequence sees all its keys: it equals the
    decode kernel's output for that query (both within the tolerance of the
    oracle, and close to each other)."""
    torch = torch_cuda
    rng = np.random.default_rng(1300)
    kl, ql = [1000, 64, 513], [48, 64, 1]
    case, cu, q = _make(rng, Hq=16, Hkv=2, D=128, bs=16, kv_dtype="bf16", klens=kl, qlens=ql)
    got = _gpu(torch, case, cu, q, True)
    last = cu[1:] - 1
    qd = torch.from_numpy(np.ascontiguousarray(q[last])).to("cuda")
    dec = pa.paged_attn_decode(qd, _pool(torch, case, case.k_store), _pool(torch, case, case.v_store),
                               torch.from_numpy(case.block_table).to("cuda"),
                               torch.from_numpy(case.seqlens).to("cuda"), case.scale)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy().astype(np.float64)
    assert np.abs(got[last] - dec).max() <= 3e-3


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (256, 12, 2)])
def test_prefill_bf16_q_and_out(torch_cuda, D, Hq, Hkv, dt):
    """q given in bf16 and out written in bf16 (PA_FLAG_QO_BF16): q is drawn as
    values bf16 holds exactly, so the oracle sees the same queries the kernel
    reads. bf16 q over bf16 K gives exact products (the scale is applied to the
    fp32 scores); over fp16 K, and fp32 q over either, Q' goes in hi + lo
    parts with the scale folded in, so the two calls differ in rounding only:
    each is within the K/V tolerance of the oracle, the bf16 output plus half a
    bf16 ulp."""
    from paged_gqa_decode_block_amd import workload as W

    torch = torch_cuda
    rng = np.random.default_rng(1301 + D + (dt == "f16"))
    case, cu, q = _make(rng, Hq=Hq, Hkv=Hkv, D=D, bs=16, kv_dtype=dt, klens=[200, 50, 700],
                        qlens=[40, 50, 33])
    q = W.from_storage(W.to_storage(q, "bf16"), "bf16").astype(np.float32)
    want = _oracle(case, cu, q, True)
    got16 = _gpu(torch, case, cu, q, True, bf16=True)
    got32 = _gpu(torch, case, cu, q, True)
    assert np.isfinite(got16).all() and np.isfinite(got32).all()
    assert (np.abs(got16 - want) <= 3e-3 + np.abs(want) * 2.0 ** -8).all()
    assert np.abs(got32 - want).max() <= 3e-3


@pytest.mark.parametrize("bf16_q", [False, True], ids=["q32", "q16"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_prefill_peaked_softmax(torch_cuda, dt, bf16_q):
    """Scores with a standard deviation of 8 (K and V drawn with std 2, scale
    4/sqrt(d)): a few keys carry nearly all the weight, the case where the
    16-bit rounding of the probabilities weighs most. Within the K/V tolerance
    of the oracle (plus half a bf16 ulp for bf16 out)."""
    from paged_gqa_decode_block_amd import workload as W

    torch = torch_cuda
    rng = np.random.default_rng(1310 + (dt == "f16") + 2 * bf16_q)
    case, cu, q = _make(rng, Hq=16, Hkv=2, D=128, bs=16, kv_dtype=dt, klens=[37, 500, 1200],
                        qlens=[37, 64, 100], scale=4.0 / np.sqrt(128), kv_std=2.0)
    if bf16_q:
        q = W.from_storage(W.to_storage(q, "bf16"), "bf16").astype(np.float32)
    want = _oracle(case, cu, q, True)
    got = _gpu(torch, case, cu, q, True, bf16=bf16_q)
    assert np.isfinite(got).all()
    tol = 3e-3 + (np.abs(want) * 2.0 ** -8 if bf16_q else 0.0)
    err = np.abs(got - want)
    print(f"peaked softmax {dt} {'bf16' if bf16_q else 'fp32'} q: max-abs error {err.max():.3e}")
    assert (err <= tol).all()


def _set_v(case, b, t, h, dim, value):
    """Set V[token t of sequence b, KV head h, dim] in the pool (HND)."""
    from paged_gqa_decode_block_amd import workload as W

    blk = 1 + int(case.block_table[b, t // case.bs])
    case.v_store[blk, h, t % case.bs, dim] = W.to_storage(np.array([value], np.float32),
                                                          case.kv_dtype)[0]


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("bf16_q", [False, True], ids=["q32", "q16"])
def test_prefill_v_beyond_f16_range(torch_cuda, bf16_q, D):
    """bf16 V values that fp16 cannot hold: tokens in 32-token tiles 2 and 6
    of sequence 0 hold +-3e5 and -65536 (the smallest bf16 magnitude beyond
    fp16's range), tile 4 holds 65280 (the largest bf16 value fp16 holds), and
    sequence 1 is untouched. Every output is finite and within 3e-3 of the
    oracle relative to max(1, |want|) (plus half a bf16 ulp for bf16 out).
    At d = 256 with bf16 q the LDS tiles hold 64 tokens, so the second pass
    also folds tiles from their second half."""
    from paged_gqa_decode_block_amd import workload as W

    torch = torch_cuda
    rng = np.random.default_rng(1320 + bf16_q + 2 * (D == 256))
    case, cu, q = _make(rng, Hq=8, Hkv=2, D=D, bs=16, kv_dtype="bf16", klens=[300, 200],
                        qlens=[40, 20])
    _set_v(case, 0, 70, 0, 5, 3.0e5)
    _set_v(case, 0, 71, 1, 100, -3.0e5)
    _set_v(case, 0, 130, 1, 7, 65280.0)
    _set_v(case, 0, 200, 0, 64, -65536.0)
    if bf16_q:
        q = W.from_storage(W.to_storage(q, "bf16"), "bf16").astype(np.float32)
    want = _oracle(case, cu, q, True)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = _gpu(torch, case, cu, q, True, bf16=bf16_q, status=status)
    assert int(status.item()) == 0
    assert np.isfinite(got).all()
    assert np.abs(want).max() > 100.0            # the large values do reach the output
    err = np.abs(got - want) / np.maximum(1.0, np.abs(want))
    print(f"V beyond fp16: max error relative to max(1, |want|) {err.max():.3e}")
    assert err.max() <= 3e-3 + (2.0 ** -8 if bf16_q else 0.0)


def test_prefill_reports_rows_beyond_max_seqlen_q(torch_cuda):
    torch = torch_cuda
    rng = np.random.default_rng(1302)
    case, cu, q = _make(rng, Hq=4, Hkv=2, D=64, bs=16, kv_dtype="bf16", klens=[100, 100],
                        qlens=[40, 10])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = _gpu(torch, case, cu, q, True, max_q=16, status=status)   # sequence 0 has 40 rows
    assert int(status.item()) & pa.PA_STATUS_BAD_SEQLEN
    want = _oracle(case, cu, q, True)
    assert np.abs(got[:16] - want[:16]).max() <= 3e-3                # the rows that fit
    assert np.abs(got[40:] - want[40:]).max() <= 3e-3                # sequence 1 complete


@pytest.mark.parametrize("k", [1, 2])
def test_prefill_workloads_whole_output(torch_cuda, k):
    """The bench's chunked-prefill workloads at full size, in the bench's launch
    configuration (causal, max_seqlen_q the longest chunk): every (row, head)
    output against the oracle."""
    from paged_gqa_decode_block_amd import workload as W

    torch = torch_cuda
    c, cu, q = W.make_prefill(k)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = _gpu(torch, c, cu, q, True, max_q=int(np.diff(cu).max()), status=status)
    assert int(status.item()) == 0
    assert np.isfinite(got).all()
    want = O.paged_attn_prefill(q, c.k_pool, c.v_pool, c.block_table, cu, c.seqlens, c.scale,
                                causal=True, kv_dtype=c.kv_dtype, block_size=c.bs,
                                num_kv_heads=c.Hkv, layout=c.layout)
    err = float(np.abs(got - want).max())
    print(f"prefill workload {k}: max-abs error {err:.3e} over {got.size} values")
    assert err <= 3e-3


def _split_case(rng):
    """24 sequences at d = 256, G = 6, 64 query rows at most: 96 (sequence, KV
    head) pairs of 3 work items each, 36 per XCD against the 32 workgroups an
    XCD holds at once, so the last 4 items of every XCD (sequences 20-23) run
    as two halves of their keys. Sequence 20 (20 keys) and 22 (33 keys) leave
    the second half of their items without a key tile; 21 has 400 keys."""
    klens = rng.integers(64, 400, size=24).astype(np.int32)
    klens[20:] = [20, 400, 33, 64]
    qlens = np.minimum(klens, 64)
    return _make(rng, Hq=24, Hkv=4, D=256, bs=16, kv_dtype="bf16", klens=klens, qlens=qlens)


def _counters_zero(torch, case, q, max_q):
    """The cached key-split workspace's arrival counters are zero again."""
    desc = pa.desc_for(torch.empty(1, case.Hq, case.D, device="cuda"), _pool(torch, case, case.k_store),
                       _pool(torch, case, case.v_store),
                       torch.from_numpy(case.block_table).to("cuda"), layout=case.layout)
    desc.batch = case.B
    zb = pa.prefill_workspace_zeroed_bytes(desc, max_q)
    ws = pa.prefill_workspace_for(desc, max_q, torch.device("cuda"))
    torch.cuda.synchronize()
    return zb > 0 and ws is not None and int(ws[:zb].count_nonzero().item()) == 0


@pytest.mark.parametrize("bf16_q", [False, True], ids=["q32", "q16"])
def test_prefill_key_split(torch_cuda, bf16_q):
    """Split work items against the oracle, element by element, twice in a row
    (the arrival counters are left zero for the next call), and against the
    same launch with every item whole (no workspace)."""
    from paged_gqa_decode_block_amd import workload as W

    torch = torch_cuda
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split plan of this batch assumes 256 compute units")
    rng = np.random.default_rng(1330 + bf16_q)
    case, cu, q = _split_case(rng)
    if bf16_q:
        q = W.from_storage(W.to_storage(q, "bf16"), "bf16").astype(np.float32)
    want = _oracle(case, cu, q, True)
    tol = 3e-3 + (np.abs(want) * 2.0 ** -8 if bf16_q else 0.0)
    outs = []
    for split in (True, True, False):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        got = _gpu(torch, case, cu, q, True, max_q=64, status=status, bf16=bf16_q, split=split)
        assert int(status.item()) == 0
        assert np.isfinite(got).all()
        err = np.abs(got - want)
        print(f"key split {split}: max-abs error {err.max():.3e}")
        assert (err <= tol).all(), split
        outs.append(got)
    assert _counters_zero(torch, case, q, 64)
    # the merged halves and the whole items differ in rounding only (which
    # half merges may differ between calls): fp32 sums, plus one bf16 ulp of
    # the output for bf16 out
    ulp = np.abs(want) * 2.0 ** -7 if bf16_q else 0.0
    assert (np.abs(outs[0] - outs[2]) <= 1e-3 + ulp).all()
    assert (np.abs(outs[0] - outs[1]) <= 1e-5 + ulp).all()


@pytest.mark.parametrize("bf16_q", [False, True], ids=["q32", "q16"])
def test_prefill_key_split_v_beyond_f16_range(torch_cuda, bf16_q):
    """A split item whose first half holds a bf16 V value beyond fp16's range
    (that half folds its tiles again as bf16) and whose second half does not:
    the merge of the two is within the oracle's tolerance relative to
    max(1, |want|) (plus half a bf16 ulp for bf16 out). With bf16 q the
    halves are cut at a 64-token tile."""
    from paged_gqa_decode_block_amd import workload as W

    torch = torch_cuda
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split plan of this batch assumes 256 compute units")
    rng = np.random.default_rng(1340)
    case, cu, q = _split_case(rng)
    _set_v(case, 21, 40, 1, 17, 3.0e5)      # sequence 21, key 40: the first half
    _set_v(case, 21, 41, 3, 200, -65536.0)
    if bf16_q:
        q = W.from_storage(W.to_storage(q, "bf16"), "bf16").astype(np.float32)
    want = _oracle(case, cu, q, True)
    got = _gpu(torch, case, cu, q, True, max_q=64, bf16=bf16_q)
    assert np.isfinite(got).all()
    assert np.abs(want).max() > 100.0
    err = np.abs(got - want) / np.maximum(1.0, np.abs(want))
    print(f"key split, V beyond fp16: max error relative to max(1, |want|) {err.max():.3e}")
    assert err.max() <= 3e-3 + (2.0 ** -8 if bf16_q else 0.0)
    assert _counters_zero(torch, case, q, 64)


SPLIT_CASES = [
    # name, B, Hq, Hkv, D, K/V dtype, bf16 q, causal: each plan splits the last
    # round (256 compute units): d = 128 bf16 q over bf16 K/V holds 96
    # workgroups per XCD at once, 14 x 8 pairs x 16 items = 224 per XCD = 2 x 96
    # + 32; over fp16 K/V 64 at once, 5 x 8 pairs -> 80 = 64 + 16; d = 256
    # without the causal mask as in test_prefill_key_split
    ("d128_bf16_q16", 14, 64, 8, 128, "bf16", True, True),
    ("d128_f16_q16", 5, 64, 8, 128, "f16", True, True),
    ("d128_bf16_q32", 5, 64, 8, 128, "bf16", False, True),
    ("d256_full", 24, 24, 4, 256, "bf16", True, False),
]


@pytest.mark.parametrize("idx", range(len(SPLIT_CASES)), ids=[c[0] for c in SPLIT_CASES])
def test_prefill_key_split_shapes(torch_cuda, idx):
    """The key split on other head sizes, K/V and q types and without the
    causal mask: 256 query rows per sequence (at most), key counts in 256..700,
    against the oracle, and the workspace's counters zero again after."""
    from paged_gqa_decode_block_amd import workload as W

    torch = torch_cuda
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split plans of these batches assume 256 compute units")
    name, B, Hq, Hkv, D, dt, bf16_q, causal = SPLIT_CASES[idx]
    rng = np.random.default_rng(1350 + idx)
    klens = rng.integers(256, 700, size=B).astype(np.int32)
    qmax = 64 if D == 256 else 256
    qlens = np.minimum(klens, qmax)
    case, cu, q = _make(rng, Hq=Hq, Hkv=Hkv, D=D, bs=16, kv_dtype=dt, klens=klens, qlens=qlens)
    desc = pa.desc_for(torch.empty(1, Hq, D, device="cuda",
                                   dtype=torch.bfloat16 if bf16_q else torch.float32),
                       _pool(torch, case, case.k_store), _pool(torch, case, case.v_store),
                       torch.from_numpy(case.block_table).to("cuda"))
    desc.batch = B
    assert pa.prefill_workspace_size(desc, qmax) > 0, name
    if bf16_q:
        q = W.from_storage(W.to_storage(q, "bf16"), "bf16").astype(np.float32)
    want = _oracle(case, cu, q, causal)
    got = _gpu(torch, case, cu, q, causal, max_q=qmax, bf16=bf16_q)
    assert np.isfinite(got).all()
    tol = 3e-3 + (np.abs(want) * 2.0 ** -8 if bf16_q else 0.0)
    err = np.abs(got - want)
    print(f"{name}: max-abs error {err.max():.3e}")
    assert (err <= tol).all(), name
    ws = pa.prefill_workspace_for(desc, qmax, torch.device("cuda"))
    zb = pa.prefill_workspace_zeroed_bytes(desc, qmax)
    torch.cuda.synchronize()
    assert int(ws[:zb].count_nonzero().item()) == 0
