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
from util_cases import paged_case, run_oracle

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
    """Every kernel that can run this case: VALU always; for 16-bit K/V the
    one-workgroup-per-partition MFMA kernel and, for block_size >= 16 and at
    most 1024 sequences, the persistent streaming MFMA kernel."""
    if case.kv_dtype == "f32":
        return ["valu"]
    out = ["valu", "mfma_grid"]
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


# --- the five workloads ------------------------------------------------------

_CASES = {}


def config_case(k):
    if k not in _CASES:
        _CASES.clear()  # keep one large workload in host memory at a time
        _CASES[k] = W.make_config(k)
    return _CASES[k]


def sample_pairs(case, n, rng):
    """All (b, h) pairs when few, else a sample that covers every sequence, every
    KV head, the shortest and the longest sequence."""
    if case.B * case.Hq <= n:
        return None
    b = np.concatenate([np.arange(case.B), rng.integers(0, case.B, size=max(0, n - case.B))])
    h = rng.integers(0, case.Hq, size=b.size)
    h[: case.Hkv] = np.arange(case.Hkv) * case.G
    b[: case.Hkv] = int(np.argmax(case.seqlens))
    b[case.Hkv: 2 * case.Hkv] = int(np.argmin(case.seqlens))
    h[case.Hkv: 2 * case.Hkv] = np.arange(case.Hkv) * case.G + case.G - 1
    return np.stack([b[:n], h[:n]], axis=1)


@pytest.mark.parametrize("k,path", [(1, "valu")] + [
    (k, path) for k in (2, 3, 4, 5) for path in ("mfma_stream", "mfma_grid", "valu")])
def test_config_matches_oracle(torch_cuda, k, path):
    case = config_case(k)
    rng = np.random.default_rng(k)
    pairs = sample_pairs(case, 192, rng)
    want = run_oracle(case, pairs=pairs)
    got = run_gpu(torch_cuda, case, path=path)
    assert np.isfinite(got).all()
    if pairs is not None:
        got = got[pairs[:, 0], pairs[:, 1]]
    err = np.abs(got - want).max()
    print(f"config {k} {path}: max-abs error {err:.3e}")
    assert err <= TOL[case.kv_dtype]


def test_config5_shared_blocks_cacheable_loads(torch_cuda):
    """The prefix-shared workload with the shared-blocks flag (cacheable K/V
    loads) and the library's own partition choice."""
    case = config_case(5)
    rng = np.random.default_rng(55)
    pairs = sample_pairs(case, 192, rng)
    want = run_oracle(case, pairs=pairs)
    for path in ("mfma_stream", "auto"):
        got = run_gpu(torch_cuda, case, path=path, partition_size=0, kv_shared=True)
        assert np.isfinite(got).all()
        assert np.abs(got[pairs[:, 0], pairs[:, 1]] - want).max() <= 3e-3, path


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
    pairs = np.stack([np.arange(1000), rng.integers(0, 4, size=1000)], axis=1)
    want = run_oracle(case, pairs=pairs)
    for ps in (32, 64):
        got = run_gpu(torch_cuda, case, path="mfma_stream", partition_size=ps)
        assert np.abs(got[pairs[:, 0], pairs[:, 1]] - want).max() <= 3e-3, ps


def test_stream_kernel_continuation_chains(torch_cuda):
    """The 100K-token workload with 4096- and 8192-token partitions: a wave's
    share (about 24 chunks) is much shorter than a partition (256 or 512
    chunks), so each partition is pieced together from ten or more waves'
    continuation states."""
    case = config_case(3)
    want = run_oracle(case)
    for ps in (4096, 8192):
        got = run_gpu(torch_cuda, case, path="mfma_stream", partition_size=ps)
        assert np.isfinite(got).all()
        assert np.abs(got - want).max() <= 3e-3, ps


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
