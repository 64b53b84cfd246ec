"""Pins for the fp64 CPU oracle, against things other than the oracle itself.

Each test names what fixes the expected value: the docs page's worked example,
a contiguous brute-force attention, a closed form, or an invariant of softmax
attention. Together they are meant to catch a dropped term, a wrong sign, a
wrong index or stride, a wrong head map and reads of unattended slots.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from paged_gqa_decode_block_amd import workload as W
from util_cases import brute_force, paged_case, run_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p5_decode_example.json")


# --- decoders ---------------------------------------------------------------

def test_f16_decoder_all_bit_patterns():
    """The oracle's binary16 decoder equals numpy's float16 widening on all 2^16 patterns."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = O.decode16(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_bf16_decoder_all_bit_patterns():
    """The oracle's bfloat16 decoder equals torch's own bfloat16 -> float64
    widening (an implementation independent of the oracle's) on all 2^16
    patterns: zeros of both signs, subnormals, normals, infinities and NaNs."""
    import torch

    bits = np.arange(1 << 16, dtype=np.uint16)
    got = O.decode16(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))   # -0.0 stays negative
    # spot values from the bfloat16 layout: 1 sign, 8 exponent (bias 127), 7 fraction bits
    spots = {0x3F80: 1.0, 0xC000: -2.0, 0x3F81: 1.0 + 2.0 ** -7, 0x0001: 2.0 ** -133,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x0080: 2.0 ** -126, 0x7F80: math.inf}
    for b, v in spots.items():
        assert O.decode16(np.array([b], dtype=np.uint16), "bf16")[0] == v, hex(b)


# --- the docs page's worked example ----------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_p5_token_to_slot_map():
    """Cached tokens land in the blocks the page names, in order, with the page's counts,
    and the slot after the last cached token is the page's next-token slot."""
    g = _golden()
    table = np.array(g["block_table"], dtype=np.int32)
    bs = g["block_size"]
    for b, L in enumerate(g["cache_seqlens"]):
        blocks, counts = [], []
        for t in range(L):
            phys, off, rc = O.token_slot(table, bs, 8, b, t)
            assert rc == 0
            if not blocks or blocks[-1] != phys:
                blocks.append(phys)
                counts.append(0)
            assert off == counts[-1], "offsets within a block run 0, 1, 2, ..."
            counts[-1] += 1
        assert blocks == g["cached_in_blocks"][b]
        assert counts == g["tokens_per_block"][b]
        phys, off, rc = O.token_slot(table, bs, 8, b, L)
        assert rc == 0 and [phys, off] == g["next_token_slot"][b]
    # an entry of -1 is unassigned: the oracle refuses it
    _, _, rc = O.token_slot(table, bs, 8, 0, 32)
    assert rc != 0


def _p5_case(rng, poison=True):
    g = _golden()
    bs, NB, D, Hq, Hkv = g["block_size"], 8, 64, 4, 2
    store = lambda: rng.standard_normal((NB + 1, Hkv, bs, D)).astype(np.float32)
    k_store, v_store = store(), store()
    holds = np.zeros((NB, bs), dtype=bool)
    for blocks, counts in zip(g["cached_in_blocks"], g["tokens_per_block"]):
        for blk, n in zip(blocks, counts):
            holds[blk, :n] = True
    if poison:
        for s in (k_store, v_store):
            s[0] = np.nan
            blks, offs = np.nonzero(~holds)
            s[1:][blks, :, offs, :] = np.nan
    case = W.Case(
        name="p5", kv_dtype="f32", B=3, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, MBS=g["max_blocks_per_seq"],
        seqlens=np.array(g["cache_seqlens"], dtype=np.int32),
        block_table=np.array(g["block_table"], dtype=np.int32),
        q=rng.standard_normal((3, Hq, D)).astype(np.float32), k_store=k_store, v_store=v_store,
        scale=0.125)
    return case, holds


def test_p5_reads_exactly_the_cached_slots():
    """NaN in every slot the page does not place a cached token in: output finite.
    Changing any slot the page does place a token in changes the output."""
    rng = np.random.default_rng(5)
    case, holds = _p5_case(rng)
    out = run_oracle(case)
    assert np.isfinite(out).all()
    blks, offs = np.nonzero(holds)
    for i in rng.choice(len(blks), size=12, replace=False):
        v2 = case.v_store.copy()
        v2[1 + blks[i], :, offs[i], :] += 1.0
        c2 = W.Case(**{**case.__dict__, "v_store": v2})
        assert not np.array_equal(run_oracle(c2), out)


# --- brute force --------------------------------------------------------------

SHAPES = [
    # B, Hq, Hkv, D, bs, dtype, layout, seqlens
    (3, 4, 2, 64, 32, "f32", "HND", [30, 32, 70]),
    (2, 14, 2, 16, 16, "f16", "NHD", [1, 47]),
    (4, 6, 1, 8, 4, "bf16", "HND", [5, 4, 1, 13]),
    (2, 8, 8, 32, 1, "f32", "NHD", [7, 3]),
    (3, 8, 2, 24, 8, "bf16", "NHD", [17, 8, 9]),
    (1, 7, 7, 40, 16, "f16", "HND", [33]),
]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_matches_contiguous_brute_force(idx):
    B, Hq, Hkv, D, bs, dt, layout, L = SHAPES[idx]
    rng = np.random.default_rng(100 + idx)
    case, Kc, Vc = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=dt, seqlens=L,
                              layout=layout)
    got = run_oracle(case)
    want = brute_force(case.q, Kc, Vc, case.scale, Hq // Hkv)
    assert np.abs(got - want).max() <= 1e-12


def test_wide_scores_match_brute_force():
    """Large-magnitude scores (max subtraction matters) still match."""
    rng = np.random.default_rng(11)
    case, Kc, Vc = paged_case(rng, B=2, Hq=4, Hkv=2, D=16, bs=4, kv_dtype="f32", seqlens=[9, 14],
                              scale=3.0)
    got = run_oracle(case)
    want = brute_force(case.q, Kc, Vc, case.scale, 2)
    assert np.abs(got - want).max() <= 1e-12


# --- special cases and closed forms ----------------------------------------

def test_single_token_returns_that_v_row_exactly():
    rng = np.random.default_rng(1)
    case, Kc, Vc = paged_case(rng, B=3, Hq=6, Hkv=3, D=32, bs=8, kv_dtype="bf16", seqlens=[1, 1, 1])
    out = run_oracle(case)
    for b in range(3):
        for h in range(6):
            assert np.array_equal(out[b, h], Vc[b][h // 2][0])


def test_identical_v_rows_return_that_row():
    rng = np.random.default_rng(2)
    case, Kc, Vc = paged_case(rng, B=2, Hq=4, Hkv=2, D=16, bs=4, kv_dtype="f32", seqlens=[11, 6])
    v = rng.standard_normal(16).astype(np.float32)
    for b in range(2):
        for j in range(-(-int(case.seqlens[b]) // 4)):
            case.v_store[1 + case.block_table[b, j]] = v  # every slot of the block, all heads
    out = run_oracle(case)
    assert np.allclose(out, np.broadcast_to(v.astype(np.float64), out.shape), rtol=1e-14, atol=0)


def test_block_relabeling_is_bitwise_invariant():
    """Permute physical ids and rewrite the table to match: output bitwise unchanged."""
    rng = np.random.default_rng(3)
    case, _, _ = paged_case(rng, B=3, Hq=8, Hkv=2, D=32, bs=4, kv_dtype="f16", seqlens=[9, 1, 16])
    out = run_oracle(case)
    perm = rng.permutation(case.NB)
    k2 = case.k_store.copy()
    v2 = case.v_store.copy()
    k2[1 + perm] = case.k_store[1:]
    v2[1 + perm] = case.v_store[1:]
    t2 = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    c2 = W.Case(**{**case.__dict__, "k_store": k2, "v_store": v2, "block_table": t2})
    assert np.array_equal(run_oracle(c2), out)


@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_uniform_scores_give_the_mean_of_v(how):
    rng = np.random.default_rng(4)
    case, Kc, Vc = paged_case(rng, B=2, Hq=4, Hkv=2, D=24, bs=8, kv_dtype="bf16", seqlens=[13, 40],
                              scale=0.0 if how == "zero_scale" else None)
    if how == "zero_q":
        case.q[:] = 0
    out = run_oracle(case)
    for b in range(2):
        for h in range(4):
            assert np.allclose(out[b, h], Vc[b][h // 2].mean(axis=0), rtol=0, atol=1e-13)


def test_two_tokens_closed_form():
    """L = 2: out = sigma(s0 - s1) v0 + (1 - sigma(s0 - s1)) v1."""
    rng = np.random.default_rng(6)
    case, Kc, Vc = paged_case(rng, B=1, Hq=2, Hkv=1, D=16, bs=1, kv_dtype="f32", seqlens=[2])
    out = run_oracle(case)
    for h in range(2):
        s = [case.scale * float(np.dot(case.q[0, h].astype(np.float64), Kc[0][0][t])) for t in range(2)]
        a = 1.0 / (1.0 + math.exp(-(s[0] - s[1])))
        want = a * Vc[0][0][0] + (1 - a) * Vc[0][0][1]
        assert np.abs(out[0, h] - want).max() <= 1e-14


def test_v_shift_equivariance():
    """out(V + 1 c^T) = out(V) + c, since the weights sum to one. V is first snapped
    to multiples of 2^-10 and c is integer, so the shifted pool is exact in fp32."""
    rng = np.random.default_rng(7)
    case, _, _ = paged_case(rng, B=2, Hq=4, Hkv=2, D=16, bs=4, kv_dtype="f32", seqlens=[10, 3])
    case.v_store[:] = np.round(case.v_store * 1024) / 1024  # NaN poison stays NaN
    c = rng.integers(-4, 5, size=16).astype(np.float32)
    out = run_oracle(case)
    c2 = W.Case(**{**case.__dict__, "v_store": (case.v_store + c).astype(np.float32)})
    out2 = run_oracle(c2)
    assert np.abs(out2 - (out + c.astype(np.float64))).max() <= 1e-12


def test_gqa_head_map_is_h_div_g():
    """V of KV head j filled with the constant j: query head h reads h // G."""
    rng = np.random.default_rng(8)
    Hq, Hkv = 12, 3
    case, _, _ = paged_case(rng, B=2, Hq=Hq, Hkv=Hkv, D=8, bs=4, kv_dtype="f32", seqlens=[9, 5])
    for j in range(Hkv):
        case.v_store[1:, j] = np.where(np.isnan(case.v_store[1:, j]), np.nan, float(j))
    out = run_oracle(case)
    for h in range(Hq):
        assert np.allclose(out[:, h], h // (Hq // Hkv), rtol=0, atol=1e-13)


def test_empty_sequence_gives_zero():
    rng = np.random.default_rng(9)
    case, _, _ = paged_case(rng, B=3, Hq=4, Hkv=2, D=8, bs=4, kv_dtype="f32", seqlens=[5, 0, 2])
    out = run_oracle(case)
    assert np.all(out[1] == 0) and np.isfinite(out).all()


# --- masking and errors -------------------------------------------------------

def test_poisoned_unread_slots_never_read():
    """Unread slots NaN: output finite and bitwise equal to the same case with those
    slots holding ordinary numbers."""
    case = W.build_case("c2_small", B=8, Hq=14, Hkv=2, D=64, bs=16, kv_dtype="f16", MBS=40,
                        seqlen_sampler=lambda r: r.integers(1, 600, size=8), spare_frac=0.2,
                        seed=77)
    out = run_oracle(case)
    assert np.isfinite(out).all()
    k2, v2 = case.k_store.copy(), case.v_store.copy()
    k2[np.isnan(W.from_storage(k2, "f16"))] = 0x3C00  # 1.0
    v2[np.isnan(W.from_storage(v2, "f16"))] = 0x4000  # 2.0
    out2 = run_oracle(W.Case(**{**case.__dict__, "k_store": k2, "v_store": v2}))
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("bad", ["minus_one_in_range", "id_ge_nb", "len_too_long", "len_negative"])
def test_invalid_inputs_are_refused(bad):
    rng = np.random.default_rng(10)
    case, _, _ = paged_case(rng, B=2, Hq=2, Hkv=1, D=8, bs=4, kv_dtype="f32", seqlens=[9, 5])
    t = case.block_table.copy()
    L = case.seqlens.copy()
    if bad == "minus_one_in_range":
        t[0, 1] = -1
    elif bad == "id_ge_nb":
        t[1, 0] = case.NB
    elif bad == "len_too_long":
        L[0] = case.MBS * case.bs + 1
    else:
        L[1] = -1
    with pytest.raises(O.OracleError):
        run_oracle(W.Case(**{**case.__dict__, "block_table": t, "seqlens": L}))


# --- the split / online algebra the GPU path relies on ----------------------

def _fold(s, v):
    """One piece, folded tile by tile with the running (m, l, acc) recurrence
    (page "v10_triton_paged_gqa", core principle; tiles of 3 tokens)."""
    m, l, acc = -math.inf, 0.0, np.zeros(v.shape[1])
    for i in range(0, len(s), 3):
        st, vt = s[i:i + 3], v[i:i + 3]
        m_new = max(m, st.max())
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        p = np.exp(st - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ vt
        m = m_new
    return m, l, acc


def _combine(a, b):
    """Max-rescaling merge of two partial states (page "Paged Attention Kernel
    Architecture for BI-V100", section 2, the compound attention_partial op)."""
    m = max(a[0], b[0])
    sa, sb = math.exp(a[0] - m), math.exp(b[0] - m)
    return m, sa * a[1] + sb * b[1], sa * a[2] + sb * b[2]


def test_split_online_combine_equals_full_softmax():
    rng = np.random.default_rng(12)
    case, Kc, Vc = paged_case(rng, B=1, Hq=2, Hkv=1, D=16, bs=4, kv_dtype="f32", seqlens=[41])
    out = run_oracle(case)
    s = case.scale * (Kc[0][0] @ case.q[0, 0].astype(np.float64))
    for cuts in ([], [7], [5, 19, 20, 33], list(range(1, 41, 4))):
        edges = [0] + cuts + [41]
        parts = [_fold(s[a:b], Vc[0][0][a:b]) for a, b in zip(edges[:-1], edges[1:])]
        for order in (parts, parts[::-1], [parts[i] for i in rng.permutation(len(parts))]):
            st = order[0]
            for p in order[1:]:
                st = _combine(st, p)
            assert np.abs(st[2] / st[1] - out[0, 0]).max() <= 1e-12


# --- plumbing -----------------------------------------------------------------

def test_pair_subset_and_thread_count_do_not_change_bits():
    rng = np.random.default_rng(13)
    case, _, _ = paged_case(rng, B=4, Hq=6, Hkv=2, D=32, bs=8, kv_dtype="bf16", seqlens=[30, 1, 64, 17])
    full1 = run_oracle(case, nthreads=1)
    full8 = run_oracle(case, nthreads=8)
    assert np.array_equal(full1, full8)
    pairs = np.array([[2, 5], [0, 0], [3, 1]])
    sub = run_oracle(case, pairs=pairs)
    for i, (b, h) in enumerate(pairs):
        assert np.array_equal(sub[i], full1[b, h])
