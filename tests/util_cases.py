"""Test-side helpers: paging contiguous K/V into a pool, and a contiguous
brute-force attention used to pin the oracle.

Nothing here is used by the GPU library or by the oracle itself.
"""
from __future__ import annotations

import math

import numpy as np

from paged_gqa_decode_block_amd import workload as W


def brute_force(q, Kc, Vc, scale, G):
    """Contiguous fp64 attention, matrix form, no block table.

    q: float [B, Hq, D]; Kc, Vc: lists (per sequence) of float64 [Hkv, L_b, D].
    Returns float64 [B, Hq, D] (zeros for an empty sequence).
    """
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        if Kc[b].shape[1] == 0:
            continue
        for h in range(Hq):
            kh = Kc[b][h // G]
            vh = Vc[b][h // G]
            s = float(scale) * (kh @ q[b, h].astype(np.float64))
            w = np.exp(s - s.max())
            out[b, h] = (w @ vh) / w.sum()
    return out


def paged_case(rng, *, B, Hq, Hkv, D, bs, kv_dtype, seqlens, layout="HND", spare=3, kv_std=1.0,
               scale=None, q=None):
    """Draw contiguous K/V per sequence, cut each sequence into pages of ``bs``
    tokens and place the pages on randomly chosen distinct physical blocks.

    Returns (case, Kc, Vc) where Kc/Vc are the contiguous float64 values (after
    rounding to the storage type) that the paged pool holds.
    """
    seqlens = np.asarray(seqlens, dtype=np.int32)
    pages = [-(-int(L) // bs) for L in seqlens]
    NB = sum(pages) + spare
    MBS = max(1, max(pages) + int(rng.integers(0, 3)))
    ids = rng.permutation(NB).astype(np.int32)
    table = np.full((B, MBS), -1, dtype=np.int32)
    pool_dtype = np.float32 if kv_dtype == "f32" else np.uint16
    shape = (NB + 1, Hkv, bs, D) if layout == "HND" else (NB + 1, bs, Hkv, D)
    nan = np.float32(np.nan) if kv_dtype == "f32" else np.uint16(0x7FC0 if kv_dtype == "bf16" else 0x7E00)
    k_store = np.full(shape, nan, dtype=pool_dtype)
    v_store = np.full(shape, nan, dtype=pool_dtype)
    if q is None:
        q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    Kc, Vc = [], []
    pos = 0
    for b in range(B):
        L = int(seqlens[b])
        kb = W.to_storage((rng.standard_normal((Hkv, L, D)) * kv_std).astype(np.float32), kv_dtype)
        vb = W.to_storage((rng.standard_normal((Hkv, L, D)) * kv_std).astype(np.float32), kv_dtype)
        Kc.append(W.from_storage(kb, kv_dtype).astype(np.float64))
        Vc.append(W.from_storage(vb, kv_dtype).astype(np.float64))
        n = pages[b]
        table[b, :n] = ids[pos:pos + n]
        pos += n
        for j in range(n):
            lo, hi = j * bs, min(L, (j + 1) * bs)
            blk = 1 + table[b, j]
            if layout == "HND":
                k_store[blk, :, : hi - lo, :] = kb[:, lo:hi, :]
                v_store[blk, :, : hi - lo, :] = vb[:, lo:hi, :]
            else:
                k_store[blk, : hi - lo, :, :] = kb[:, lo:hi, :].transpose(1, 0, 2)
                v_store[blk, : hi - lo, :, :] = vb[:, lo:hi, :].transpose(1, 0, 2)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    case = W.Case(
        name="paged_random", kv_dtype=kv_dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, MBS=MBS,
        seqlens=seqlens, block_table=table, q=q, k_store=k_store, v_store=v_store, layout=layout,
        scale=float(np.float32(scale)),
    )
    return case, Kc, Vc


def shared_prefix_case(rng, *, Hq, Hkv, D, bs, kv_dtype, families, layout="HND", mismatch=None,
                       spare=2):
    """A batch whose sequences come in families sharing leading blocks.

    ``families``: list of (prefix_blocks, [member lengths]). Each member lists
    its family's prefix blocks first (as many as its length reaches), then
    blocks of its own. ``mismatch`` = (family, member, block): that member's
    prefix block is replaced by a private copy (same values, another physical
    block), which ends what its group can share. Physical blocks are placed at
    random; every token slot no listing attends is NaN-poisoned.
    """
    lens, rows, content = [], [], {}  # content: logical block -> source logical block
    nlog = 0
    for pb, members in families:
        pre = list(range(nlog, nlog + pb))
        nlog += pb
        for L in members:
            n = -(-int(L) // bs)
            row = pre[:min(pb, n)] + list(range(nlog, nlog + max(0, n - pb)))
            nlog += max(0, n - pb)
            rows.append(row)
            lens.append(int(L))
    if mismatch is not None:
        fi, mi, j = mismatch
        b = sum(len(m) for _, m in families[:fi]) + mi
        content[nlog] = rows[b][j]
        rows[b][j] = nlog
        nlog += 1
    NB = nlog + spare
    perm = rng.permutation(NB).astype(np.int32)       # logical -> physical
    B = len(rows)
    MBS = max(1, max(len(r) for r in rows) + int(rng.integers(0, 3)))
    table = np.full((B, MBS), -1, dtype=np.int32)
    for b, row in enumerate(rows):
        table[b, :len(row)] = perm[row]
    # tokens attended in each physical block (max over its listings)
    att = np.zeros(NB, dtype=np.int64)
    for b, row in enumerate(rows):
        for j, lb in enumerate(row):
            att[perm[lb]] = max(att[perm[lb]], min(bs, lens[b] - j * bs))
    pool_dtype = np.float32 if kv_dtype == "f32" else np.uint16
    shape = (NB + 1, Hkv, bs, D) if layout == "HND" else (NB + 1, bs, Hkv, D)
    nan = np.float32(np.nan) if kv_dtype == "f32" else np.uint16(0x7FC0 if kv_dtype == "bf16" else 0x7E00)
    k_store = np.full(shape, nan, dtype=pool_dtype)
    v_store = np.full(shape, nan, dtype=pool_dtype)
    vals = {}
    for lb in range(nlog):
        src = content.get(lb, lb)
        if src not in vals:
            vals[src] = tuple(W.to_storage(rng.standard_normal((Hkv, bs, D)).astype(np.float32), kv_dtype)
                              for _ in range(2))
    for lb in range(nlog):
        kb, vb = vals[content.get(lb, lb)]
        blk, n = 1 + perm[lb], int(att[perm[lb]])
        if layout == "HND":
            k_store[blk, :, :n] = kb[:, :n]
            v_store[blk, :, :n] = vb[:, :n]
        else:
            k_store[blk, :n] = kb[:, :n].transpose(1, 0, 2)
            v_store[blk, :n] = vb[:, :n].transpose(1, 0, 2)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    case = W.Case(
        name="shared_prefix", kv_dtype=kv_dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, MBS=MBS,
        seqlens=np.asarray(lens, dtype=np.int32), block_table=table, q=q, k_store=k_store,
        v_store=v_store, layout=layout, scale=float(np.float32(1.0 / math.sqrt(D))),
    )
    return case


def run_oracle(case, **kw):
    from oracle import oracle as O

    return O.paged_attn_decode(
        case.q, case.k_pool, case.v_pool, case.block_table, case.seqlens, case.scale,
        kv_dtype=case.kv_dtype, block_size=case.bs, num_kv_heads=case.Hkv, layout=case.layout, **kw)


# One generated workload (and its whole-batch oracle output) is kept at a time:
# the large ones take seconds to draw and gigabytes of host memory.
_CONFIG = {}


def config_case(k):
    """Decode workload k (``workload.make_config``), cached while it is the
    most recently requested one."""
    if _CONFIG.get("k") != k:
        _CONFIG.clear()
        _CONFIG["k"] = k
        _CONFIG["case"] = W.make_config(k)
    return _CONFIG["case"]


def config_oracle(k):
    """The oracle's output for every (sequence, query head) of workload k."""
    case = config_case(k)
    if "want" not in _CONFIG:
        _CONFIG["want"] = run_oracle(case)
    return _CONFIG["want"]
