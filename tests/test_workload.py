"""The seeded generator builds the five workloads as described, deterministically."""
import json
import os

import numpy as np
import pytest

from paged_gqa_decode_block_amd import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p5_decode_example.json")


def test_bf16_rounding_is_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)  # bf16 spacing in [1, 2)
    x = np.array([one, one + ulp / 2, one + ulp * 1.5, one + ulp / 2 + np.float32(2.0 ** -20),
                  -one - ulp / 2], dtype=np.float32)
    got = W.from_storage(W.to_storage(x, "bf16"), "bf16")
    want = np.array([1.0, 1.0, 1.0 + 2 * ulp, 1.0 + ulp, -1.0], dtype=np.float32)
    assert np.array_equal(got, want)


def test_config1_is_the_docs_example():
    g = json.load(open(GOLDEN))
    c = W.make_config(1)
    assert c.seqlens.tolist() == g["cache_seqlens"]
    assert c.block_table.tolist() == g["block_table"]
    assert (c.NB, c.MBS, c.bs, c.D, c.Hq, c.Hkv, c.kv_dtype) == (8, 4, 32, 64, 4, 2, "f32")
    assert c.scale == 0.125
    # poison: block 2 offsets 30-31, block 1 (assigned, unused), block 6 offsets 6-31,
    # unreferenced blocks 4 and 7, and the guard
    k = c.k_pool
    assert np.isnan(k[2, :, 30:]).all() and np.isfinite(k[2, :, :30]).all()
    assert np.isnan(k[1]).all() and np.isnan(k[4]).all() and np.isnan(k[7]).all()
    assert np.isnan(k[6, :, 6:]).all() and np.isfinite(k[6, :, :6]).all()
    assert np.isfinite(k[0]).all() and np.isfinite(k[3]).all() and np.isfinite(k[5]).all()
    assert np.isnan(c.k_store[0]).all() and np.isnan(c.v_store[0]).all()


def test_determinism_same_seed_same_bits():
    a = W.make_config(2)
    b = W.make_config(2)
    for f in ("seqlens", "block_table", "q", "k_store", "v_store"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=False) or \
            np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8))
    c = W.make_config(2, seed=5)
    assert not np.array_equal(a.q, c.q)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_permutation_placement(k):
    c = W.make_config(k, tables_only=True)
    used = np.concatenate([c.block_table[b, : -(-int(L) // c.bs)] for b, L in enumerate(c.seqlens)])
    assert len(np.unique(used)) == len(used), "no block is shared"
    assert used.min() >= 0 and used.max() < c.NB
    for b, L in enumerate(c.seqlens):
        n = -(-int(L) // c.bs)
        assert (c.block_table[b, n:] == -1).all()
    if k == 4:
        assert c.NB == int(np.ceil(1.1 * len(used)))
        assert c.seqlens.min() >= 1024 and c.seqlens.max() <= 32768
    else:
        assert c.NB == len(used)
    if k == 2:
        assert c.seqlens.min() >= 512 and c.seqlens.max() <= 4096
    if k == 3:
        assert c.seqlens.tolist() == [100000] and c.NB == 6250


def test_config5_prefix_families():
    c = W.make_config(5, tables_only=True)
    assert (c.B, c.Hq, c.Hkv, c.D, c.bs, c.MBS) == (256, 32, 8, 128, 32, 252)
    assert c.seqlens[-1] == 1 and (c.seqlens[:-1] >= 2049).all() and (c.seqlens[:-1] <= 8048).all()
    for f in range(16):
        rows = c.block_table[16 * f:16 * f + 16]
        full = rows[:15] if f == 15 else rows
        assert (full[:, :64] == full[0, :64]).all(), "members share the 64 prefix blocks"
    last = c.block_table[-1]
    assert last[0] == c.block_table[-2, 0] and (last[1:] == -1).all()
    ref = c.ref_count
    fam15 = c.block_table[240, :64]
    assert ref[fam15[0]] == 16 and (ref[fam15[1:]] == 15).all()
    assert (ref[c.block_table[0, :64]] == 16).all()
    assert ref.max() == 16 and (ref >= 1).all()
    # -1 padding after each row's last listed block
    for b, L in enumerate(c.seqlens):
        n = -(-int(L) // c.bs)
        assert (c.block_table[b, :n] >= 0).all() and (c.block_table[b, n:] == -1).all()


def test_unread_slots_poisoned_read_slots_finite():
    c = W.build_case("t", B=5, Hq=4, Hkv=2, D=16, bs=8, kv_dtype="bf16",
                     seqlen_sampler=lambda r: r.integers(1, 50, size=5), spare_frac=0.3, seed=3)
    read = W.read_mask(c.block_table, c.seqlens, c.NB, c.bs)
    kf = W.from_storage(c.k_pool, "bf16")
    for blk in range(c.NB):
        for off in range(c.bs):
            assert np.isfinite(kf[blk, :, off]).all() == read[blk, off]
            assert np.isnan(kf[blk, :, off]).all() == (not read[blk, off])


def test_nhd_layout_same_tables_token_major_strides():
    a = W.build_case("t", B=2, Hq=4, Hkv=2, D=8, bs=4, kv_dtype="f16", seqlens=[5, 9], seed=9)
    b = W.build_case("t", B=2, Hq=4, Hkv=2, D=8, bs=4, kv_dtype="f16", seqlens=[5, 9], seed=9,
                     layout="NHD")
    assert np.array_equal(a.block_table, b.block_table)
    assert a.strides() == (64, 32, 8) and b.strides() == (64, 8, 16)


@pytest.mark.parametrize("dtype,x", [(np.uint16, 8), (np.float32, 4)])
def test_xpacked_layout_is_the_pages_indexing(dtype, x):
    """to_xpacked against the layout's definition, element by element: K element
    (blk, h, t, i) sits at [blk, h, i // x, t, i % x] of [NB, H, d/x, bs, x]
    (x = 16 bytes / element) and V element (blk, h, t, i) at [blk, h, i, t]."""
    rng = np.random.default_rng(7)
    NB, H, bs, D = 3, 2, 8, 32
    pool = rng.integers(0, 60000, size=(NB, H, bs, D)).astype(dtype)
    kx, vx = W.to_xpacked(pool, "k"), W.to_xpacked(pool, "v")
    assert kx.shape == (NB, H, D // x, bs, x) and vx.shape == (NB, H, D, bs)
    assert kx.flags["C_CONTIGUOUS"] and vx.flags["C_CONTIGUOUS"]
    for blk in range(NB):
        for h in range(H):
            for t in range(bs):
                for i in range(D):
                    assert kx[blk, h, i // x, t, i % x] == pool[blk, h, t, i]
                    assert vx[blk, h, i, t] == pool[blk, h, t, i]
