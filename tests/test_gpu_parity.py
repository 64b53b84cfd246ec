"""GPU parity: the HIP path against the fp64 CPU oracle, element by element.

Tolerance (max-abs): 1e-5 for fp32 K/V, 3e-3 for fp16/bf16 K/V (fp32
accumulation). Masking is checked by NaN poison in every unattended slot and a
NaN guard block in front of the pool: any read of them would turn the output
NaN. Every call goes through the C ABI (libpagedattn.so).
"""
import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from paged_gqa_decode_block_amd import workload as W
from util_cases import config_case, config_oracle, paged_case, run_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3, "bf16": 3e-3}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()  # fail loudly if the HIP library is missing
    return torch


def to_device(torch, case):
    def pool(store):
        if case.kv_dtype == "f32":
            t = torch.from_numpy(np.ascontiguousarray(store))
        else:
            t = torch.from_numpy(np.ascontiguousarray(store).view(np.int16))
            t = t.view(torch.bfloat16 if case.kv_dtype == "bf16" else torch.float16)
        return t.to("cuda")[1:]  # the guard block stays in front of the pool

    return dict(
        q=torch.from_numpy(case.q).to("cuda"),
        k=pool(case.k_store),
        v=pool(case.v_store),
        table=torch.from_numpy(case.block_table).to("cuda"),
        seqlens=torch.from_numpy(case.seqlens).to("cuda"),
    )


def run_gpu(torch, case, dev=None, *, path="auto", partition_size=None, status=None,
            kv_shared=False):
    dev = dev or to_device(torch, case)
    ps = case.partition_size if partition_size is None else partition_size
    out = pa.paged_attn_decode(dev["q"], dev["k"], dev["v"], dev["table"], dev["seqlens"],
                               case.scale, layout=case.layout, partition_size=ps, path=path,
                               status=status, kv_shared=kv_shared)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def paths_for(case):
    """Every kernel that can run this case: VALU for groups of up to 8 heads;
    for 16-bit K/V the one-workgroup-per-partition MFMA kernel and, for
    block_size >= 16 and at most 1024 sequences, the persistent streaming MFMA
    kernel."""
    if case.kv_dtype == "f32":
        return ["valu"]
    out = (["valu"] if case.Hq // case.Hkv <= 8 else []) + ["mfma_grid"]
    if case.bs >= 16 and case.B <= 1024:
        out.append("mfma_stream")
    return out


# --- small cases spanning several tiles, ragged tails, edge lengths ---------

SMALL = [
    # name, B, Hq, Hkv, D, bs, dtype, layout, seqlens, partition
    ("p5_like_f32", 3, 4, 2, 64, 32, "f32", "HND", [30, 32, 70], 32),
    ("f32_d128_g8", 2, 16, 2, 128, 16, "f32", "NHD", [1, 200], 64),
    ("f32_d256_g3", 2, 6, 2, 256, 8, "f32", "HND", [77, 33], 32),
    ("f16_d64_g7", 3, 14, 2, 64, 16, "f16", "HND", [513, 1, 100], 128),
    ("bf16_d128_g8", 4, 32, 4, 128, 16, "bf16", "HND", [31, 32, 33, 700], 64),
    ("bf16_d256_g6", 1, 24, 4, 256, 16, "bf16", "HND", [1000], 512),
    ("bf16_d128_g4_bs32", 3, 16, 4, 128, 32, "bf16", "NHD", [2049, 5, 64], 512),
    ("f16_d128_g1", 2, 4, 4, 128, 4, "f16", "NHD", [45, 130], 32),
    ("bf16_d64_g2_bs1", 2, 4, 2, 64, 1, "bf16", "HND", [40, 3], 32),
    ("bf16_d128_g5_bs64", 2, 10, 2, 128, 64, "bf16", "HND", [300, 64], 96),
    ("f16_d256_g8_part2048", 2, 16, 2, 256, 16, "f16", "HND", [2500, 2048], 2048),
    ("bf16_empty_and_one", 4, 8, 2, 128, 16, "bf16", "HND", [0, 1, 0, 17], 32),
    # d = 256 (a pair of waves per share in the streaming kernel): token-major
    # rows, the largest group, 32-token blocks; and one head per group in fp16
    ("bf16_d256_g16_nhd_bs32", 2, 32, 2, 256, 32, "bf16", "NHD", [1500, 47], 512),
    ("f16_d256_g1", 3, 2, 2, 256, 16, "f16", "HND", [33, 700, 1], 64),
    # the largest block: one 1024-token block holds a whole short sequence
    ("bf16_d128_g2_bs1024", 3, 4, 2, 128, 1024, "bf16", "HND", [1500, 1024, 3], 512),
]


@pytest.mark.parametrize("idx", range(len(SMALL)), ids=[s[0] for s in SMALL])
def test_small_cases_match_oracle(torch_cuda, idx):
    name, B, Hq, Hkv, D, bs, dt, layout, L, part = SMALL[idx]
    rng = np.random.default_rng(500 + idx)
    case, _, _ = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=dt, seqlens=L,
                            layout=layout, spare=4)
    want = run_oracle(case)
    dev = to_device(torch_cuda, case)
    for path in paths_for(case):
        for ps in (part, 0):
            got = run_gpu(torch_cuda, case, dev, path=path, partition_size=ps)
            assert np.isfinite(got).all(), (path, ps)
            err = np.abs(got - want).max()
            assert err <= TOL[dt], (name, path, ps, err)


def test_g16_on_matrix_cores(torch_cuda):
    rng = np.random.default_rng(77)
    case, _, _ = paged_case(rng, B=2, Hq=32, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[333, 90])
    want = run_oracle(case)
    for path in ("mfma_grid", "mfma_stream"):
        got = run_gpu(torch_cuda, case, path=path, partition_size=64)
        assert np.abs(got - want).max() <= 3e-3, path


def test_peaked_softmax_keeps_tolerance(torch_cuda):
    """Few dominant tokens (scale 4): the hi/lo split of Q and P keeps the MFMA
    products accurate where a single bf16 P would not be."""
    rng = np.random.default_rng(78)
    for dt in ("bf16", "f16"):
        case, _, _ = paged_case(rng, B=2, Hq=8, Hkv=2, D=128, bs=16, kv_dtype=dt,
                                seqlens=[2, 37], scale=4.0 / np.sqrt(128), kv_std=2.0)
        want = run_oracle(case)
        for path in paths_for(case):
            got = run_gpu(torch_cuda, case, path=path, partition_size=32)
            assert np.abs(got - want).max() <= 3e-3, (dt, path)


# --- the five workloads at full size are in test_gpu_configs.py ---------------

def test_config1_combine_path(torch_cuda):
    """Config 1 with 32-token partitions: sequence 2 spans three partitions."""
    case = W.make_config(1)
    want = run_oracle(case)
    got = run_gpu(torch_cuda, case, path="valu", partition_size=32)
    assert np.abs(got - want).max() <= 1e-5


# --- masking, invalid input, invariants ------------------------------------

def test_invalid_entries_are_skipped_and_reported(torch_cuda):
    torch = torch_cuda
    rng = np.random.default_rng(90)
    case, _, _ = paged_case(rng, B=3, Hq=8, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[70, 40, 20])
    case.block_table[0, 1] = -1          # unassigned entry inside the attended range
    case.block_table[1, 0] = case.NB     # beyond the pool
    for path in paths_for(case):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        got = run_gpu(torch, case, path=path, partition_size=32, status=status)
        assert int(status.item()) & pa.PA_STATUS_BAD_BLOCK
        assert np.isfinite(got).all()
    case.block_table[0, 1] = case.block_table[0, 0]
    case.block_table[1, 0] = case.block_table[1, 1]
    case.seqlens[2] = case.MBS * case.bs + 5   # too long: clamped and reported
    for path in paths_for(case):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        run_gpu(torch, case, path=path, partition_size=32, status=status)
        assert int(status.item()) & pa.PA_STATUS_BAD_SEQLEN, path


def test_block_relabeling_and_reruns_are_bitwise_identical(torch_cuda):
    torch = torch_cuda
    rng = np.random.default_rng(91)
    case, _, _ = paged_case(rng, B=3, Hq=12, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[300, 17, 129])
    perm = rng.permutation(case.NB)
    k2, v2 = case.k_store.copy(), case.v_store.copy()
    k2[1 + perm] = case.k_store[1:]
    v2[1 + perm] = case.v_store[1:]
    t2 = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    c2 = W.Case(**{**case.__dict__, "k_store": k2, "v_store": v2, "block_table": t2})
    for path in paths_for(case):
        a = run_gpu(torch, case, path=path, partition_size=64)
        b = run_gpu(torch, case, path=path, partition_size=64)
        c = run_gpu(torch, c2, path=path, partition_size=64)
        assert np.array_equal(a, b) and np.array_equal(a, c), path


def test_single_token_returns_v_row(torch_cuda):
    rng = np.random.default_rng(92)
    case, Kc, Vc = paged_case(rng, B=4, Hq=8, Hkv=2, D=256, bs=16, kv_dtype="bf16",
                              seqlens=[1, 1, 1, 1])
    for path in paths_for(case):
        got = run_gpu(torch_cuda, case, path=path)
        for b in range(4):
            for h in range(8):
                assert np.array_equal(got[b, h], Vc[b][h // 4][0]), path


# --- the streaming kernel's work split -----------------------------------------

STREAM_CASES = [
    # name, B, Hq, Hkv, D, bs, dtype, seqlens, partition
    ("many_partitions_per_wave", 3, 16, 2, 128, 16, "bf16", [3000, 77, 1500], 32),
    ("empty_between", 6, 8, 4, 64, 16, "f16", [0, 300, 0, 0, 45, 1], 64),
    ("d256_short_parts", 2, 12, 2, 256, 32, "bf16", [900, 2000], 64),
    ("partial_last_chunk", 2, 8, 1, 128, 64, "bf16", [33, 1025], 512),
    # one partition per sequence, each split over ~16 waves (500 chunks, 31 waves)
    ("single_partition_many_waves", 2, 8, 1, 128, 16, "bf16", [4000, 3990], 4096),
    # nothing to attend: zeros from the combine
    ("all_empty", 3, 8, 2, 128, 16, "bf16", [0, 0, 0], 64),
    # 4800 chunks: 300 waves' worth, rounded down to a multiple of the compute units
    ("waves_rounded_to_cus", 1, 8, 2, 128, 16, "bf16", [38400], 512),
]


@pytest.mark.parametrize("idx", range(len(STREAM_CASES)), ids=[s[0] for s in STREAM_CASES])
def test_stream_kernel_work_split(torch_cuda, idx):
    name, B, Hq, Hkv, D, bs, dt, L, part = STREAM_CASES[idx]
    rng = np.random.default_rng(700 + idx)
    case, _, _ = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=dt, seqlens=L, spare=2)
    want = run_oracle(case)
    got = run_gpu(torch_cuda, case, path="mfma_stream", partition_size=part)
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() <= 3e-3


def test_stream_kernel_thousand_sequences(torch_cuda):
    """1000 sequences: the item prefix spans all 16 windows of the scan."""
    rng = np.random.default_rng(800)
    L = rng.integers(0, 120, size=1000)
    case, _, _ = paged_case(rng, B=1000, Hq=4, Hkv=2, D=64, bs=16, kv_dtype="bf16", seqlens=L)
    want = run_oracle(case)
    for ps in (32, 64):
        got = run_gpu(torch_cuda, case, path="mfma_stream", partition_size=ps)
        assert np.isfinite(got).all(), ps
        assert np.abs(got - want).max() <= 3e-3, ps


@pytest.mark.parametrize("B", [1024, 1025])
def test_batch_at_and_past_the_stream_limit(torch_cuda, B):
    """1024 sequences fill all 16 windows of the streaming kernel's scan; one
    more and the library picks the grid kernel (the streaming kernel, asked
    for by name, is refused before any launch)."""
    rng = np.random.default_rng(810 + B)
    L = rng.integers(0, 100, size=B)
    case, _, _ = paged_case(rng, B=B, Hq=4, Hkv=2, D=64, bs=16, kv_dtype="bf16", seqlens=L)
    want = run_oracle(case)
    dev = to_device(torch_cuda, case)
    paths = ["auto", "mfma_grid"] + (["mfma_stream"] if B <= 1024 else [])
    for path in paths:
        got = run_gpu(torch_cuda, case, dev, path=path, partition_size=64)
        assert np.isfinite(got).all(), path
        assert np.abs(got - want).max() <= 3e-3, path
    if B > 1024:
        with pytest.raises(RuntimeError):
            run_gpu(torch_cuda, case, dev, path="mfma_stream", partition_size=64)


def test_stream_kernel_continuation_chains(torch_cuda):
    """The 100K-token workload with 4096- and 8192-token partitions: a wave's
    share (about 24 chunks) is much shorter than a partition (256 or 512
    chunks), so each partition is pieced together from ten or more waves'
    continuation states."""
    case = config_case(3)
    want = config_oracle(3)
    for ps in (4096, 8192):
        got = run_gpu(torch_cuda, case, path="mfma_stream", partition_size=ps)
        assert np.isfinite(got).all()
        assert np.abs(got - want).max() <= 3e-3, ps


@pytest.mark.parametrize("path", ["mfma_stream", "mfma_grid", "valu"])
def test_poisoned_workspace_is_never_used(torch_cuda, path):
    """Every byte of the workspace set to 0xFF before each call (NaN in every
    float slot, -1 in every link): the combine reads partition slots up to the
    workspace's row length before it knows a sequence's own partition count,
    and must drop the stale ones. Sequences of 0, 1, a few and many partitions
    share one batch, so most rows hold slots past their own count."""
    torch = torch_cuda
    rng = np.random.default_rng(910)
    L = [0, 1, 33, 700, 5000, 64, 2049]
    case, _, _ = paged_case(rng, B=len(L), Hq=16, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=L, spare=3)
    want = run_oracle(case)
    dev = to_device(torch, case)
    for ps in (32, 64, 512):
        desc = pa.desc_for(dev["q"], dev["k"], dev["v"], dev["table"], partition_size=ps,
                           path=path)
        ws = torch.full((max(pa.workspace_size(desc), 256),), 0xFF, dtype=torch.uint8,
                        device="cuda")
        for rep in range(2):
            ws.fill_(0xFF)
            out = pa.paged_attn_decode(dev["q"], dev["k"], dev["v"], dev["table"],
                                       dev["seqlens"], case.scale, partition_size=ps, path=path,
                                       workspace=ws)
            got = out.cpu().numpy().astype(np.float64)
            assert np.isfinite(got).all(), (path, ps, rep)
            assert np.abs(got - want).max() <= 3e-3, (path, ps, rep)


@pytest.mark.parametrize("D,Hq,Hkv,part", [(256, 24, 4, 512), (128, 16, 2, 64)])
def test_stream_kernel_one_sequence_table_fill(torch_cuda, D, Hq, Hkv, part):
    """One long sequence whose block table it fills exactly, to one token or
    one block short, or to half: the streaming kernel's shares then fall on
    stream ends in different places; unread slots are NaN, so any read of a
    wrong table entry or of a slot past the length would show."""
    torch = torch_cuda
    bs = 16
    for i, (L, mbs) in enumerate([(12800, 800), (12799, 800), (12784, 800), (6400, 800)]):
        rng = np.random.default_rng(950 + i)
        case, _, _ = paged_case(rng, B=1, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype="bf16",
                                seqlens=[L], spare=mbs)
        pages = -(-L // bs)
        table = np.full((1, mbs), -1, dtype=np.int32)
        table[0, :pages] = case.block_table[0, :pages]
        case.block_table = table
        case.MBS = mbs
        want = run_oracle(case)
        got = run_gpu(torch, case, path="mfma_stream", partition_size=part)
        assert np.isfinite(got).all(), (L, mbs)
        assert np.abs(got - want).max() <= 3e-3, (L, mbs)


def test_partition_then_combine_phase_equals_decode(torch_cuda):
    """The two phases called one after the other give the one-call result bit
    for bit (same workspace, same stream)."""
    torch = torch_cuda
    rng = np.random.default_rng(93)
    case, _, _ = paged_case(rng, B=3, Hq=16, Hkv=2, D=128, bs=16, kv_dtype="bf16",
                            seqlens=[3000, 77, 1500])
    dev = to_device(torch, case)
    args = (dev["q"], dev["k"], dev["v"], dev["table"], dev["seqlens"], case.scale)
    for path in ("mfma_stream", "mfma_grid"):
        full = pa.paged_attn_decode(*args, partition_size=64, path=path)
        out = torch.zeros_like(full)
        pa.paged_attn_decode(*args, out, partition_size=64, path=path, phase="partition")
        pa.paged_attn_decode(*args, out, partition_size=64, path=path, phase="combine")
        torch.cuda.synchronize()
        assert torch.equal(out, full), path


# --- the decode step with the new token (append in place), and graph replay -----

def _append_case(rng, *, kv_dtype="bf16", layout="HND", L0=(100, 31, 200), steps=4, B=3, Hq=8,
                 Hkv=2, D=128, bs=16):
    """A paged case whose tables already map `steps` more tokens per sequence; the
    slots of those future tokens hold NaN until an append writes them."""
    final = [int(x) + steps for x in L0]
    case, _, _ = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=kv_dtype, seqlens=final,
                            layout=layout)
    nan = np.float32(np.nan) if kv_dtype == "f32" else np.uint16(0x7FC0 if kv_dtype == "bf16" else 0x7E00)
    for b in range(B):
        for t in range(L0[b], final[b]):
            _slot(case, b, t)[0][...] = nan
            _slot(case, b, t)[1][...] = nan
    return W.Case(**{**case.__dict__, "seqlens": np.asarray(L0, dtype=np.int32)})


def _slot(case, b, t):
    """Views of token t of sequence b in the host K and V stores ([H_kv, d])."""
    blk = 1 + case.block_table[b, t // case.bs]
    off = t % case.bs
    if case.layout == "HND":
        return case.k_store[blk, :, off, :], case.v_store[blk, :, off, :]
    return case.k_store[blk, off, :, :], case.v_store[blk, off, :, :]


def _new_token(torch, rng, case):
    """Step inputs: q (float32) and k_new / v_new in the cache's storage type, on
    host and device."""
    q = rng.standard_normal((case.B, case.Hq, case.D)).astype(np.float32)
    kn = W.to_storage(rng.standard_normal((case.B, case.Hkv, case.D)).astype(np.float32), case.kv_dtype)
    vn = W.to_storage(rng.standard_normal((case.B, case.Hkv, case.D)).astype(np.float32), case.kv_dtype)

    def dev(a):
        if case.kv_dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.view(torch.bfloat16 if case.kv_dtype == "bf16" else torch.float16).to("cuda")

    return q, kn, vn, torch.from_numpy(q).to("cuda"), dev(kn), dev(vn)


def _append_host(case, q, kn, vn):
    """The host-side step: write the new token, return the case to attend (L + 1)."""
    for b in range(case.B):
        ks, vs = _slot(case, b, int(case.seqlens[b]))
        ks[...] = kn[b]
        vs[...] = vn[b]
    return W.Case(**{**case.__dict__, "q": q, "seqlens": case.seqlens + 1})


@pytest.mark.parametrize("kv_dtype,layout", [("bf16", "HND"), ("f16", "NHD"), ("f32", "HND")])
def test_decode_append_matches_oracle(torch_cuda, kv_dtype, layout):
    """Two decode steps, each appending the new token in place and attending it:
    every kernel path against the oracle on the updated cache, and the cache slot
    holds exactly the appended rows (NaN poison in the future slots would show a
    read before the write)."""
    torch = torch_cuda
    for path in paths_for(_append_case(np.random.default_rng(0), kv_dtype=kv_dtype, layout=layout)):
        rng = np.random.default_rng(95)
        case = _append_case(rng, kv_dtype=kv_dtype, layout=layout)
        dev = to_device(torch, case)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        for step in range(2):
            q, kn, vn, qd, knd, vnd = _new_token(torch, rng, case)
            ref = _append_host(case, q, kn, vn)
            want = run_oracle(ref)
            got = pa.paged_attn_decode_append(qd, knd, vnd, dev["k"], dev["v"], dev["table"],
                                              dev["seqlens"], case.scale, layout=layout,
                                              partition_size=64, path=path, status=status)
            torch.cuda.synchronize()
            got = got.cpu().numpy().astype(np.float64)
            assert np.isfinite(got).all(), (path, step)
            assert np.abs(got - want).max() <= TOL[kv_dtype], (path, step)
            pool_k = dev["k"].cpu().numpy() if kv_dtype == "f32" else dev["k"].cpu().view(torch.int16).numpy().view(np.uint16)
            for b in range(case.B):
                t = int(case.seqlens[b])
                blk, off = case.block_table[b, t // case.bs], t % case.bs
                row = pool_k[blk, :, off, :] if layout == "HND" else pool_k[blk, off, :, :]
                assert np.array_equal(row.view(np.uint8), np.ascontiguousarray(kn[b]).view(np.uint8))
            dev["seqlens"] += 1
            case = W.Case(**{**ref.__dict__, "seqlens": ref.seqlens})
        assert int(status.item()) == 0, path


def test_decode_append_graph_replay(torch_cuda):
    """The append + decode step captured once in a HIP graph and replayed for four
    decode steps: inputs are updated in place between replays (new q and K/V rows
    copied in, cache lengths advanced by eager work), and every replay matches the
    oracle on the cache as it then stands."""
    torch = torch_cuda
    rng = np.random.default_rng(96)
    case = _append_case(rng, steps=4)
    dev = to_device(torch, case)
    q_s = torch.zeros(case.B, case.Hq, case.D, dtype=torch.float32, device="cuda")
    kn_s = torch.zeros(case.B, case.Hkv, case.D, dtype=torch.bfloat16, device="cuda")
    vn_s = torch.zeros_like(kn_s)
    out_s = torch.zeros_like(q_s)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (dev["k"], dev["v"], dev["table"], dev["seqlens"], case.scale)
    # a plain decode first: creates the cached workspace outside the capture
    pa.paged_attn_decode(q_s, *args, out_s, partition_size=64)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.paged_attn_decode_append(q_s, kn_s, vn_s, *args, out_s, partition_size=64, status=status)
    torch.cuda.synchronize()
    for step in range(4):
        q, kn, vn, qd, knd, vnd = _new_token(torch, rng, case)
        q_s.copy_(qd)
        kn_s.copy_(knd)
        vn_s.copy_(vnd)
        ref = _append_host(case, q, kn, vn)
        want = run_oracle(ref)
        g.replay()
        torch.cuda.synchronize()
        got = out_s.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), step
        assert np.abs(got - want).max() <= 3e-3, step
        dev["seqlens"] += 1   # eager work between replays
        torch.cuda.synchronize()
        case = W.Case(**{**ref.__dict__, "seqlens": ref.seqlens})
    assert int(status.item()) == 0


# --- the block manager's copy-on-write on the device ---------------------------

def test_copy_on_write_with_block_manager(torch_cuda):
    """Two sequences share three blocks (the last one partly filled) through the
    block manager and both append a different token at position 40. The first
    appender gets a fresh copy of the shared block (paged_attn_copy_blocks on the
    device), the second then owns the original; each sequence attends its own
    new token, against the oracle."""
    torch = torch_cuda
    rng = np.random.default_rng(97)
    Hq, Hkv, D, bs, L, NB = 8, 2, 128, 16, 40, 8
    bm = pa.BlockManager(NB, bs)
    bm.allocate_blocks(0, 3)
    bm.share_prefix(0, 1, 3)
    k_store = np.full((NB + 1, Hkv, bs, D), 0x7FC0, dtype=np.uint16)   # bf16 NaN
    v_store = k_store.copy()
    kc = W.to_storage(rng.standard_normal((Hkv, L, D)).astype(np.float32), "bf16")
    vc = W.to_storage(rng.standard_normal((Hkv, L, D)).astype(np.float32), "bf16")
    for j, blk in enumerate(bm.sequence_blocks(0)):
        lo, hi = j * bs, min(L, (j + 1) * bs)
        k_store[1 + blk, :, : hi - lo, :] = kc[:, lo:hi, :]
        v_store[1 + blk, :, : hi - lo, :] = vc[:, lo:hi, :]
    kd = torch.from_numpy(k_store.view(np.int16)).view(torch.bfloat16).to("cuda")[1:]
    vd = torch.from_numpy(v_store.view(np.int16)).view(torch.bfloat16).to("cuda")[1:]
    pairs = [r for r in (bm.append_slot(0, L), bm.append_slot(1, L)) if r is not None]
    assert len(pairs) == 1 and bm.sequence_blocks(1)[2] == pairs[0][0]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32, device="cuda"), status=status)
    for src, dst in pairs:  # the host mirror of the copy
        k_store[1 + dst] = k_store[1 + src]
        v_store[1 + dst] = v_store[1 + src]
    table = bm.block_table([0, 1], 3)
    case = W.Case(name="cow", kv_dtype="bf16", B=2, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, MBS=3,
                  seqlens=np.array([L, L], dtype=np.int32), block_table=table,
                  q=np.zeros((2, Hq, D), dtype=np.float32), k_store=k_store, v_store=v_store,
                  scale=1.0 / np.sqrt(D))
    q, kn, vn, qd, knd, vnd = _new_token(torch, rng, case)
    ref = _append_host(case, q, kn, vn)
    want = run_oracle(ref)
    for path in ("mfma_stream", "mfma_grid", "valu"):
        out = pa.paged_attn_decode_append(qd, knd, vnd, kd, vd, torch.from_numpy(table).to("cuda"),
                                          torch.from_numpy(case.seqlens).to("cuda"), case.scale,
                                          partition_size=32, path=path, status=status)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.abs(got - want).max() <= 3e-3, path
    assert int(status.item()) == 0
    assert np.abs(want[0] - want[1]).max() > 1e-3  # the two new tokens differ


# --- bf16 q and out ---------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype", ["bf16", "f16", "f32"])
def test_bf16_q_and_out(torch_cuda, kv_dtype):
    """q given in bf16 and out written in bf16 (PA_FLAG_QO_BF16): with q values
    that bf16 holds exactly, the bf16 output is the fp32 path's output rounded
    to nearest even (torch's conversion), bit for bit, on every kernel path;
    against the oracle it is within the K/V tolerance plus half a bf16 ulp."""
    torch = torch_cuda
    rng = np.random.default_rng(98)
    q = W.from_storage(W.to_storage(rng.standard_normal((3, 16, 128)).astype(np.float32), "bf16"),
                       "bf16").astype(np.float32)
    case, _, _ = paged_case(rng, B=3, Hq=16, Hkv=2, D=128, bs=16, kv_dtype=kv_dtype,
                            seqlens=[700, 1, 33], q=q)
    want = run_oracle(case)
    dev = to_device(torch, case)
    q16 = dev["q"].to(torch.bfloat16)
    args = (dev["k"], dev["v"], dev["table"], dev["seqlens"], case.scale)
    for path in paths_for(case):
        for ps in (32, 0):
            o32 = pa.paged_attn_decode(dev["q"], *args, partition_size=ps, path=path)
            o16 = pa.paged_attn_decode(q16, *args, partition_size=ps, path=path)
            torch.cuda.synchronize()
            assert o16.dtype == torch.bfloat16
            assert torch.equal(o16, o32.to(torch.bfloat16)), (path, ps)
            got = o16.float().cpu().numpy().astype(np.float64)
            assert (np.abs(got - want) <= TOL[kv_dtype] + np.abs(want) * 2.0 ** -8).all(), (path, ps)


def test_bf16_q_and_out_d256_and_merged_variant():
    """bf16 q / out at head_dim 256 (the streaming kernel's pair of waves) and
    on the single-launch merged variant: bit for bit the fp32 path's output
    rounded to bf16, and within the K/V tolerance plus half a bf16 ulp of the
    oracle."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(99)
    q = W.from_storage(W.to_storage(rng.standard_normal((3, 12, 256)).astype(np.float32), "bf16"),
                       "bf16").astype(np.float32)
    case, _, _ = paged_case(rng, B=3, Hq=12, Hkv=2, D=256, bs=16, kv_dtype="bf16",
                            seqlens=[3000, 1, 700], q=q)
    want = run_oracle(case)
    dev = to_device(torch, case)
    q16 = dev["q"].to(torch.bfloat16)
    args = (dev["k"], dev["v"], dev["table"], dev["seqlens"], case.scale)
    for path in ("mfma_stream", "mfma_grid", "mfma_fused"):
        for ps in (256, 0):
            o32 = pa.paged_attn_decode(dev["q"], *args, partition_size=ps, path=path)
            o16 = pa.paged_attn_decode(q16, *args, partition_size=ps, path=path)
            torch.cuda.synchronize()
            assert o16.dtype == torch.bfloat16
            assert torch.equal(o16, o32.to(torch.bfloat16)), (path, ps)
            got = o16.float().cpu().numpy().astype(np.float64)
            assert (np.abs(got - want) <= 3e-3 + np.abs(want) * 2.0 ** -8).all(), (path, ps)
