"""Pins of the oracle's paged varlen prefill (CPU only).

The prefill oracle shares the fp64 softmax core with the decode oracle (which
has its own pins); what is new here is the row -> sequence mapping of the
packed queries and the causal key range of each row. They are pinned by:
- the docs page's varlen worked example (row and key labels);
- an independent contiguous brute force written with an explicit mask matrix;
- the reductions to the decode (one query per sequence; no causal mask);
- closed forms and mask invariants on tiny inputs.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from paged_gqa_decode_block_amd import workload as W
from util_cases import paged_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p5_varlen_example.json")


def _prefill(case, cu, sk, q, causal, **kw):
    return O.paged_attn_prefill(q, case.k_pool, case.v_pool, case.block_table, cu, sk, case.scale,
                                causal=causal, kv_dtype=case.kv_dtype, block_size=case.bs,
                                num_kv_heads=case.Hkv, layout=case.layout, **kw)


def _brute(q, Kc, Vc, cu, sk, scale, G, causal):
    """Contiguous fp64 attention with an explicit [q_len, L] mask per sequence:
    mask[i, t] = t <= L - q_len + i (bottom-right aligned) when causal."""
    total, Hq, D = q.shape
    out = np.zeros((total, Hq, D))
    for b in range(len(sk)):
        r0, r1, L = int(cu[b]), int(cu[b + 1]), int(sk[b])
        ql = r1 - r0
        if ql == 0 or L == 0:
            continue
        mask = np.ones((ql, L), dtype=bool)
        if causal:
            mask = np.tril(mask, k=L - ql)
        for h in range(Hq):
            kh, vh = Kc[b][h // G][:L], Vc[b][h // G][:L]
            s = float(scale) * (q[r0:r1, h].astype(np.float64) @ kh.T)
            s = np.where(mask, s, -np.inf)
            for i in range(ql):
                if not mask[i].any():
                    continue
                w = np.exp(s[i] - s[i].max())
                out[r0 + i, h] = (w @ vh) / w.sum()
    return out


def _case(rng, *, B, Hq, Hkv, D, bs, kv_dtype, seqlens):
    case, Kc, Vc = paged_case(rng, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, kv_dtype=kv_dtype,
                              seqlens=seqlens)
    return case, Kc, Vc


def test_varlen_example_row_and_key_labels():
    """The page's example: rows of the packed queries map to the sequences it
    labels, and in the paged form each row sees exactly its sequence's keys:
    sequence 0 (no keys) gives zeros, and with the causal rule sequence 1's
    three queries see nothing, nothing and key 0 (its only key)."""
    g = json.load(open(GOLDEN))
    cu = np.array(g["cu_seq_lens_q"], dtype=np.int32)
    assert list(np.diff(cu)) == g["query_lengths"]
    assert list(np.diff(np.array(g["cu_seq_lens_k"]))) == g["key_lengths"]
    assert max(g["query_lengths"]) == g["max_length_q"] and max(g["key_lengths"]) == g["max_length_k"]
    assert cu[-1] == g["q_shape_tokens"] and sum(g["key_lengths"]) == g["kv_shape_tokens"]
    labels = np.searchsorted(cu, np.arange(cu[-1]), side="right") - 1
    assert list(labels) == g["query_request_index"]
    klabels = np.repeat(np.arange(3), g["key_lengths"])
    assert list(klabels) == g["key_request_index"]
    rng = np.random.default_rng(5)
    case, Kc, Vc = _case(rng, B=3, Hq=4, Hkv=2, D=64, bs=16, kv_dtype="f32", seqlens=g["key_lengths"])
    q = rng.standard_normal((int(cu[-1]), 4, 64)).astype(np.float32)
    sk = np.array(g["key_lengths"], dtype=np.int32)
    out = _prefill(case, cu, sk, q, causal=True)
    assert np.all(out[0:10] == 0.0)                         # sequence 0: no keys
    assert np.all(out[10] == 0.0) and np.all(out[11] == 0.0)
    for h in range(4):
        assert np.array_equal(out[12, h], Vc[1][h // 2][0])  # one key: exactly its V row
    # the last row of sequence 2 sees all 7 keys, like a decode query
    dec = O.paged_attn_decode(q[13:14], case.k_pool, case.v_pool, case.block_table[2:3],
                              sk[2:3], case.scale, kv_dtype="f32", block_size=16, num_kv_heads=2)
    assert np.array_equal(out[13], dec[0])
    # without the causal rule every row of sequence 1 sees its one key
    full = _prefill(case, cu, sk, q, causal=False)
    for r in (10, 11, 12):
        for h in range(4):
            assert np.array_equal(full[r, h], Vc[1][h // 2][0])


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_matches_contiguous_brute_force(causal, kv_dtype):
    rng = np.random.default_rng(11 if causal else 12)
    sk = np.array([40, 7, 0, 33, 50], dtype=np.int32)
    ql = np.array([5, 7, 3, 40, 1], dtype=np.int32)        # q_len < L, = L, > L (0 and 33 keys)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    case, Kc, Vc = _case(rng, B=5, Hq=6, Hkv=2, D=32, bs=16, kv_dtype=kv_dtype, seqlens=sk)
    q = rng.standard_normal((int(cu[-1]), 6, 32)).astype(np.float32)
    got = _prefill(case, cu, sk, q, causal=causal)
    want = _brute(q, Kc, Vc, cu, sk, case.scale, 3, causal)
    assert np.abs(got - want).max() <= 1e-12


def test_one_query_per_sequence_is_the_decode():
    rng = np.random.default_rng(13)
    sk = np.array([1, 30, 77], dtype=np.int32)
    case, _, _ = _case(rng, B=3, Hq=8, Hkv=2, D=64, bs=32, kv_dtype="bf16", seqlens=sk)
    cu = np.arange(4, dtype=np.int32)
    for causal in (True, False):
        got = _prefill(case, cu, sk, case.q, causal=causal)
        dec = O.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_table, sk, case.scale,
                                  kv_dtype="bf16", block_size=32, num_kv_heads=2)
        assert np.array_equal(got, dec)


def test_two_tokens_closed_form():
    """q_len = L = 2, causal: row 0 sees key 0 only (its V row exactly), row 1
    sees both: sigma(s0 - s1) v0 + (1 - sigma(s0 - s1)) v1."""
    rng = np.random.default_rng(14)
    case, Kc, Vc = _case(rng, B=1, Hq=2, Hkv=1, D=16, bs=16, kv_dtype="f32", seqlens=[2])
    q = rng.standard_normal((2, 2, 16)).astype(np.float32)
    cu = np.array([0, 2], dtype=np.int32)
    out = _prefill(case, cu, np.array([2], dtype=np.int32), q, causal=True)
    for h in range(2):
        k0, k1 = Kc[0][0][0], Kc[0][0][1]
        v0, v1 = Vc[0][0][0], Vc[0][0][1]
        assert np.array_equal(out[0, h], v0)
        s0 = case.scale * float(q[1, h].astype(np.float64) @ k0)
        s1 = case.scale * float(q[1, h].astype(np.float64) @ k1)
        a = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        assert np.abs(out[1, h] - (a * v0 + (1 - a) * v1)).max() <= 1e-13


def test_causal_mask_is_exact():
    """Keys after a row's position do not touch that row: overwriting every
    key/value at positions past row i's last key leaves row i bit-identical,
    while the last row (which sees them) changes."""
    rng = np.random.default_rng(15)
    L, ql = 45, 9
    case, Kc, Vc = _case(rng, B=1, Hq=4, Hkv=1, D=32, bs=16, kv_dtype="f32", seqlens=[L])
    q = rng.standard_normal((ql, 4, 32)).astype(np.float32)
    cu = np.array([0, ql], dtype=np.int32)
    sk = np.array([L], dtype=np.int32)
    base = _prefill(case, cu, sk, q, causal=True)
    i = 3
    last = L - ql + i                     # row i's last key
    k2, v2 = case.k_store.copy(), case.v_store.copy()
    for t in range(last + 1, L):
        blk = 1 + case.block_table[0, t // 16]
        k2[blk, :, t % 16, :] = 7.0
        v2[blk, :, t % 16, :] = -3.0
    c2 = W.Case(**{**case.__dict__, "k_store": k2, "v_store": v2})
    got = _prefill(c2, cu, sk, q, causal=True)
    assert np.array_equal(got[: i + 1], base[: i + 1])
    assert np.abs(got[-1] - base[-1]).max() > 1e-3
