"""Seeded synthetic decode workloads: paged K/V pools, block tables, cache lengths, queries.

This module only draws inputs and lays them out in memory. It holds none of the
attention arithmetic, so both the CPU oracle's tests and the GPU path's tests and
bench can take their inputs from it.

Layout of a case (all host numpy arrays):

* ``q``            float32 ``[B, H_q, D]``, contiguous.
* ``k_store``,
  ``v_store``      the K and V pools *with one guard block in front*. Pool block
                   ``i`` lives at storage block ``i + 1``; storage block 0 is a
                   guard filled with NaN so that a kernel that ever dereferenced a
                   ``-1`` table entry would read NaN instead of another
                   sequence's data. ``HND`` storage is ``[NB + 1, H_kv, bs, D]``
                   (each (block, head) tile contiguous), ``NHD`` storage is
                   ``[NB + 1, bs, H_kv, D]`` (token-major). Element type is
                   float32 for ``f32`` and the raw 16-bit pattern (uint16) for
                   ``f16`` / ``bf16``.
* ``block_table``  int32 ``[B, MBS]``: physical block ids in logical order, ``-1``
                   for unassigned entries (the convention of the paged-attention
                   docs page, decode path example).
* ``seqlens``      int32 ``[B]``: cached tokens per sequence.

Every pool slot that no sequence attends to (the tail of a sequence's last block,
blocks that are assigned but not yet used, spare blocks, the guard) is
overwritten with NaN ("poison"), so an output that stays finite shows that the
kernel never read it.

Configurations 1-5 follow the five decode workloads this project is measured on;
the draw order for each is: cache lengths, block placement, Q, K pool, V pool,
all from ``numpy.random.default_rng(1000 + k)`` unless another seed is given.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KV_DTYPES = ("f32", "f16", "bf16")
_ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
_NAN_BITS16 = {"f16": 0x7E00, "bf16": 0x7FC0}
_CHUNK = 1 << 25  # elements drawn per call when filling a pool


def elem_bytes(kv_dtype: str) -> int:
    return _ELEM_BYTES[kv_dtype]


def to_storage(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Round float32 values to the KV storage type, round-to-nearest-even.

    Returns float32 for ``f32`` and the 16-bit patterns (uint16) otherwise.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if kv_dtype == "f32":
        return x
    if kv_dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if kv_dtype == "bf16":
        u = x.view(np.uint32)
        # RNE on the 16 dropped bits; inputs here are always finite.
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def from_storage(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Widen stored K/V values to float32 (exact for all three storage types)."""
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if kv_dtype == "f16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float32)
    if kv_dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def _nan_value(kv_dtype: str):
    return np.float32(np.nan) if kv_dtype == "f32" else np.uint16(_NAN_BITS16[kv_dtype])


@dataclass
class Case:
    name: str
    kv_dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    MBS: int
    seqlens: np.ndarray
    block_table: np.ndarray
    q: np.ndarray
    k_store: np.ndarray
    v_store: np.ndarray
    layout: str = "HND"
    scale: float = 0.0
    partition_size: int = 512
    ref_count: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def k_pool(self) -> np.ndarray:
        """Pool view starting at physical block 0 (the guard block excluded)."""
        return self.k_store[1:]

    @property
    def v_pool(self) -> np.ndarray:
        return self.v_store[1:]

    def strides(self) -> tuple[int, int, int]:
        """(block, head, token) strides of the pools, in elements; head_dim stride is 1."""
        if self.layout == "HND":
            return (self.Hkv * self.bs * self.D, self.bs * self.D, self.D)
        return (self.bs * self.Hkv * self.D, self.D, self.Hkv * self.D)

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode call must read: 2 * H_kv * D * s * sum(L)."""
        return 2 * self.Hkv * self.D * elem_bytes(self.kv_dtype) * int(self.seqlens.astype(np.int64).sum())

    def unique_kv_bytes(self) -> int:
        """K+V bytes of the distinct pool slots attended (prefix sharing counted once)."""
        read = read_mask(self.block_table, self.seqlens, self.NB, self.bs)
        return 2 * self.Hkv * self.D * elem_bytes(self.kv_dtype) * int(read.sum())


def read_mask(block_table: np.ndarray, seqlens: np.ndarray, NB: int, bs: int) -> np.ndarray:
    """bool [NB, bs]: slots that hold some sequence's cached token.

    Built from how the tables are constructed: sequence b's j-th listed block
    holds its tokens [j*bs, (j+1)*bs), so every listed block but the last is full.
    """
    mask = np.zeros((NB, bs), dtype=bool)
    for b in range(block_table.shape[0]):
        L = int(seqlens[b])
        if L <= 0:
            continue
        nblk = -(-L // bs)
        ids = block_table[b, :nblk]
        if nblk > 1:
            mask[ids[:-1], :] = True
        mask[ids[-1], : L - (nblk - 1) * bs] = True
    return mask


def _pool_shape(layout: str, NB: int, Hkv: int, bs: int, D: int) -> tuple[int, ...]:
    if layout == "HND":
        return (NB + 1, Hkv, bs, D)
    if layout == "NHD":
        return (NB + 1, bs, Hkv, D)
    raise ValueError(f"unknown layout {layout!r}")


def to_xpacked(store: np.ndarray, which: str) -> np.ndarray:
    """The same values in the x-packed cache layout of page "Paged Attention
    Kernel Architecture for BI-V100", section 3, from an HND pool
    [NB, H_kv, bs, d]: K ("k") becomes [NB, H_kv, d/x, bs, x] with
    x = 16 bytes / element, V ("v") becomes [NB, H_kv, d, bs]. Element
    (blk, h, t, i) moves to [blk, h, i // x, t, i % x] and [blk, h, i, t]."""
    NB, H, bs, D = store.shape
    if which == "k":
        x = 16 // store.itemsize
        return np.ascontiguousarray(store.reshape(NB, H, bs, D // x, x).transpose(0, 1, 3, 2, 4))
    if which == "v":
        return np.ascontiguousarray(store.transpose(0, 1, 3, 2))
    raise ValueError(which)


def _draw_pool(rng: np.random.Generator, shape, kv_dtype: str, std: float) -> np.ndarray:
    """Fill a storage array block by block with N(0, std^2) draws rounded to kv_dtype.

    The guard block (storage block 0) is drawn too, then poisoned, so the draw
    stream does not depend on the layout.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if kv_dtype == "f32" else np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = to_storage(x, kv_dtype)
    return out.reshape(shape)


def _poison(store: np.ndarray, layout: str, read: np.ndarray, kv_dtype: str) -> None:
    nan = _nan_value(kv_dtype)
    store[0] = nan  # guard block
    blks, offs = np.nonzero(~read)
    if blks.size == 0:
        return
    pool = store[1:]
    if layout == "HND":
        pool[blks, :, offs, :] = nan
    else:
        pool[blks, offs, :, :] = nan


def _assign_by_permutation(rng, seqlens, bs, MBS, spare_frac):
    nblk = [-(-int(L) // bs) for L in seqlens]
    total = sum(nblk)
    NB = max(1, math.ceil(total * (1.0 + spare_frac))) if spare_frac > 0 else max(1, total)
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((len(seqlens), MBS), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, NB


def build_case(
    name: str,
    *,
    B: int,
    Hq: int,
    Hkv: int,
    D: int,
    bs: int,
    kv_dtype: str,
    seqlens=None,
    MBS: int | None = None,
    spare_frac: float = 0.0,
    kv_std: float = 1.0,
    q_std: float = 1.0,
    layout: str = "HND",
    seed: int = 0,
    partition_size: int = 512,
    scale: float | None = None,
    block_table=None,
    NB: int | None = None,
    seqlen_sampler=None,
    tables_only: bool = False,
) -> Case:
    """General builder used by the five configurations and by the tests.

    Either give ``seqlens`` (list/array) or ``seqlen_sampler(rng) -> array``.
    Without an explicit ``block_table`` the blocks are placed by a seeded
    permutation of a pool sized to the total (plus ``spare_frac`` spare blocks).
    """
    assert kv_dtype in KV_DTYPES and Hq % Hkv == 0
    rng = np.random.default_rng(seed)
    # 1. cache lengths
    if seqlen_sampler is not None:
        seqlens = np.asarray(seqlen_sampler(rng), dtype=np.int32)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    assert seqlens.shape == (B,)
    if MBS is None:
        MBS = max(1, -(-int(seqlens.max(initial=0)) // bs))
    # 2. block placement
    if block_table is None:
        table, NB = _assign_by_permutation(rng, seqlens, bs, MBS, spare_frac)
    else:
        table = np.asarray(block_table, dtype=np.int32)
        assert table.shape == (B, MBS) and NB is not None
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if tables_only:
        return Case(
            name=name, kv_dtype=kv_dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, MBS=MBS,
            seqlens=seqlens, block_table=table, q=None, k_store=None, v_store=None,
            layout=layout, scale=float(np.float32(scale)), partition_size=partition_size,
        )
    # 3-5. Q, K pool, V pool
    q = (rng.standard_normal(B * Hq * D, dtype=np.float32) * np.float32(q_std)).reshape(B, Hq, D)
    shape = _pool_shape(layout, NB, Hkv, bs, D)
    k_store = _draw_pool(rng, shape, kv_dtype, kv_std)
    v_store = _draw_pool(rng, shape, kv_dtype, kv_std)
    read = read_mask(table, seqlens, NB, bs)
    _poison(k_store, layout, read, kv_dtype)
    _poison(v_store, layout, read, kv_dtype)
    return Case(
        name=name, kv_dtype=kv_dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB, MBS=MBS,
        seqlens=seqlens, block_table=table, q=q, k_store=k_store, v_store=v_store,
        layout=layout, scale=float(np.float32(scale)), partition_size=partition_size,
    )


# The worked example of the paged-attention docs page (decode path): three
# sequences with 30, 32 and 70 cached tokens, blocks of 32 tokens, four table
# entries per sequence, -1 for unassigned entries.
P5_SEQLENS = [30, 32, 70]
P5_BLOCK_TABLE = [[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]]


def _loguniform_int(rng, lo, hi, n):
    x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi + 1), size=n)))
    return np.clip(x, lo, hi).astype(np.int32)


def _config5(seed: int, layout: str, tables_only: bool = False) -> Case:
    """256 sequences in 16 families; each family shares a 2048-token prefix.

    The prefix is 64 blocks of 32 tokens, listed by all 16 members of the family
    (reference count 16). Suffixes are private, U{1..6000} tokens. The last
    sequence of the last family is cut to a single cached token: its row lists
    only the family's first prefix block.
    """
    B, Hq, Hkv, D, bs, MBS = 256, 32, 8, 128, 32, 252
    fams, per_fam, prefix_blocks = 16, 16, 64
    rng = np.random.default_rng(seed)
    suffix = rng.integers(1, 6001, size=B).astype(np.int32)
    seqlens = (2048 + suffix).astype(np.int32)
    seqlens[B - 1] = 1
    suffix_blocks = [-(-int(s) // bs) for s in suffix]
    suffix_blocks[B - 1] = 0
    NB = fams * prefix_blocks + sum(suffix_blocks)
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((B, MBS), -1, dtype=np.int32)
    pos = fams * prefix_blocks
    for b in range(B):
        f = b // per_fam
        pre = perm[f * prefix_blocks:(f + 1) * prefix_blocks]
        if b == B - 1:
            table[b, 0] = pre[0]
            continue
        n = suffix_blocks[b]
        table[b, :prefix_blocks] = pre
        table[b, prefix_blocks:prefix_blocks + n] = perm[pos:pos + n]
        pos += n
    ref = np.zeros(NB, dtype=np.int32)
    for b in range(B):
        nb = -(-int(seqlens[b]) // bs)
        np.add.at(ref, table[b, :nb], 1)
    common = dict(
        name="c5_prefix_shared_bf16", kv_dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB,
        MBS=MBS, seqlens=seqlens, block_table=table, layout=layout,
        scale=float(np.float32(1.0 / math.sqrt(D))), partition_size=512, ref_count=ref,
    )
    if tables_only:
        return Case(q=None, k_store=None, v_store=None, **common)
    q = rng.standard_normal(B * Hq * D, dtype=np.float32).reshape(B, Hq, D)
    shape = _pool_shape(layout, NB, Hkv, bs, D)
    k_store = _draw_pool(rng, shape, "bf16", 1.0)
    v_store = _draw_pool(rng, shape, "bf16", 1.0)
    read = read_mask(table, seqlens, NB, bs)
    _poison(k_store, layout, read, "bf16")
    _poison(v_store, layout, read, "bf16")
    return Case(q=q, k_store=k_store, v_store=v_store, **common)


CONFIG_NAMES = {
    1: "c1_tiny_f32",
    2: "c2_qwen2_f16",
    3: "c3_qwen36_100k_bf16",
    4: "c4_large_gqa_bf16",
    5: "c5_prefix_shared_bf16",
}


def make_config(k: int, seed: int | None = None, layout: str = "HND",
                tables_only: bool = False) -> Case:
    """The five decode workloads (1-based), seeded with ``1000 + k`` by default."""
    if seed is None:
        seed = 1000 + k
    t = dict(layout=layout, seed=seed, tables_only=tables_only)
    if k == 1:
        return build_case(
            CONFIG_NAMES[1], B=3, Hq=4, Hkv=2, D=64, bs=32, kv_dtype="f32",
            seqlens=P5_SEQLENS, MBS=4, block_table=P5_BLOCK_TABLE, NB=8, scale=1.0 / 8.0, **t,
        )
    if k == 2:
        return build_case(
            CONFIG_NAMES[2], B=8, Hq=14, Hkv=2, D=64, bs=16, kv_dtype="f16", MBS=256,
            seqlen_sampler=lambda r: r.integers(512, 4097, size=8), **t,
        )
    if k == 3:
        return build_case(
            CONFIG_NAMES[3], B=1, Hq=24, Hkv=4, D=256, bs=16, kv_dtype="bf16", MBS=6250,
            seqlens=[100000], partition_size=512, **t,
        )
    if k == 4:
        return build_case(
            CONFIG_NAMES[4], B=64, Hq=64, Hkv=8, D=128, bs=16, kv_dtype="bf16", MBS=2048,
            seqlen_sampler=lambda r: _loguniform_int(r, 1024, 32768, 64), spare_frac=0.10,
            kv_std=0.5, **t,
        )
    if k == 5:
        return _config5(seed, layout, tables_only)
    raise ValueError(f"configs are numbered 1..5, got {k}")


def make_shard(n: int, seed: int | None = None, layout: str = "HND") -> Case:
    """One GPU's share when the 100K-token context of decode workload 3 is split
    by tokens over n GPUs: the same heads and pool layout (H_q 24, H_kv 4,
    d 256, bf16, blocks of 16, partitions of 512), one sequence of
    ceil(100000 / n) tokens, seeded with 1003 + 100 n."""
    if seed is None:
        seed = 1003 + 100 * n
    L = -(-100000 // n)
    return build_case(f"c3_qwen36_100k_bf16_shard_1of{n}", B=1, Hq=24, Hkv=4, D=256, bs=16,
                      kv_dtype="bf16", MBS=-(-L // 16), seqlens=[L], partition_size=512,
                      layout=layout, seed=seed)


def make_qwen2_batch(B: int, ctx: int = 512, seed: int | None = None) -> Case:
    """B Qwen2-shaped sequences (H_q 14, H_kv 2, d 64, fp16 K/V, blocks of 16)
    of ctx cached tokens each, seeded with 4000 + B: the shape of the
    batch-scaling measurements of the paged-attention-runtime design notes."""
    if seed is None:
        seed = 4000 + B
    return build_case(f"qwen2_fp16_ctx{ctx}_batch{B}", B=B, Hq=14, Hkv=2, D=64, bs=16,
                      kv_dtype="f16", MBS=-(-ctx // 16), seqlens=[ctx] * B, seed=seed)


# Chunked-prefill workloads over the same kind of paged pool: each sequence's
# cache already holds the new chunk (its last q_len tokens), and the chunk's
# queries are packed in rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (the varlen
# indexing of the paged-attention docs page).
PREFILL_NAMES = {
    1: "p1_qwen36_chunked_prefill_bf16",
    2: "p2_large_gqa_chunked_prefill_bf16",
}


def make_prefill(k: int, seed: int | None = None, layout: str = "HND"):
    """(case, cu_seqlens_q, q) for prefill workload k, seeded with 2000 + k:

    1. the 100K-token decode shape's heads (H_q 24, H_kv 4, d 256, bf16, blocks
       of 16): 4 sequences of 8192 cached tokens whose last 512 are the chunk;
    2. the 64-sequence decode shape's heads (H_q 64, H_kv 8, d 128, bf16, blocks
       of 16): 16 sequences with lengths uniform in [1024, 8192], chunks of 256.

    ``q`` is float32 [total_q, H_q, d] ~ N(0, 1), drawn after the pool.
    """
    if seed is None:
        seed = 2000 + k
    if k == 1:
        case = build_case(PREFILL_NAMES[1], B=4, Hq=24, Hkv=4, D=256, bs=16, kv_dtype="bf16",
                          seqlens=[8192] * 4, layout=layout, seed=seed)
        qlens = np.full(4, 512, dtype=np.int32)
    elif k == 2:
        case = build_case(PREFILL_NAMES[2], B=16, Hq=64, Hkv=8, D=128, bs=16, kv_dtype="bf16",
                          seqlen_sampler=lambda r: r.integers(1024, 8193, size=16), layout=layout,
                          seed=seed)
        qlens = np.minimum(256, case.seqlens).astype(np.int32)
    else:
        raise ValueError(f"prefill workloads are numbered 1..2, got {k}")
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    rng = np.random.default_rng(seed + 500)
    q = rng.standard_normal((int(cu[-1]), case.Hq, case.D), dtype=np.float32)
    return case, cu, q
