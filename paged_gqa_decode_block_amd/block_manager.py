"""Python face of the host block manager in libpagedattn.so (C ABI in
``include/paged_block_manager.h``): free list, reference counts, per-sequence
block lists, prefix sharing and copy-on-write, and the block tables that
``paged_attn_decode`` reads. ``copy_blocks`` runs the device copy that a
copy-on-write asks for."""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import PagedAttnError, load_library


class BlockManager:
    """Physical blocks 0 .. num_blocks-1 of block_size tokens, all free at start."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = load_library()
        self._h = self._lib.paged_attn_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("num_blocks must be > 0 and block_size a power of two in [1, 1024]")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if self._h:
            self._lib.paged_attn_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    def _check(self, rc: int, what: str) -> int:
        if rc < 0:
            raise PagedAttnError(rc, f"{what}: ")
        return rc

    def allocate_blocks(self, seq_id: int, n: int) -> None:
        self._check(self._lib.paged_attn_bm_allocate_blocks(self._h, seq_id, n), "allocate_blocks")

    def free_sequence(self, seq_id: int) -> None:
        self._check(self._lib.paged_attn_bm_free_sequence(self._h, seq_id), "free_sequence")

    def share_prefix(self, source: int, target: int, n_blocks: int) -> None:
        self._check(self._lib.paged_attn_bm_share_prefix(self._h, source, target, n_blocks),
                    "share_prefix")

    def cow_block(self, seq_id: int, block_index: int):
        """None when the block was already exclusive, else (src, dst): copy src's
        K/V into dst before the sequence's next read."""
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        rc = self._check(self._lib.paged_attn_bm_cow_block(
            self._h, seq_id, block_index, ctypes.byref(src), ctypes.byref(dst)), "cow_block")
        return (src.value, dst.value) if rc == 1 else None

    def append_slot(self, seq_id: int, seq_len: int):
        """Readies token seq_len's slot; None, or the (src, dst) copy it needs."""
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        rc = self._check(self._lib.paged_attn_bm_append_slot(
            self._h, seq_id, seq_len, ctypes.byref(src), ctypes.byref(dst)), "append_slot")
        return (src.value, dst.value) if rc == 1 else None

    @property
    def num_free(self) -> int:
        return self._check(self._lib.paged_attn_bm_num_free(self._h), "num_free")

    def ref_count(self, block: int) -> int:
        return self._check(self._lib.paged_attn_bm_ref_count(self._h, block), "ref_count")

    def sequence_blocks(self, seq_id: int) -> list[int]:
        n = self._check(self._lib.paged_attn_bm_sequence_blocks(self._h, seq_id, None, 0),
                        "sequence_blocks")
        out = (ctypes.c_int32 * max(n, 1))()
        self._check(self._lib.paged_attn_bm_sequence_blocks(self._h, seq_id, out, n),
                    "sequence_blocks")
        return list(out[:n])

    def block_table(self, seq_ids, max_blocks_per_seq: int) -> np.ndarray:
        """int32 [len(seq_ids), max_blocks_per_seq], -1 padded."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        table = np.empty((ids.size, max_blocks_per_seq), dtype=np.int32)
        self._check(self._lib.paged_attn_bm_block_table(
            self._h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ids.size,
            max_blocks_per_seq, table.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
            "block_table")
        return table


def copy_blocks(k_cache, v_cache, pairs, *, layout="HND", status=None, stream=None) -> None:
    """Device copy of whole blocks (every KV head) src -> dst in both pools;
    ``pairs`` is an int32 device tensor [n, 2] of (src, dst)."""
    import torch

    from . import desc_for

    lib = load_library()
    NB = k_cache.shape[0]
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise ValueError("pairs must be a contiguous int32 [n, 2] tensor")
    # a descriptor for the pools (q and the table only lend their shapes)
    Hkv = k_cache.shape[2] if layout == "NHD" else k_cache.shape[1]
    D = v_cache.shape[2] if layout == "XPACKED" else k_cache.shape[3]
    q = torch.empty(1, Hkv, D, dtype=torch.float32, device=k_cache.device)
    table = torch.empty(1, 1, dtype=torch.int32, device=k_cache.device)
    desc = desc_for(q, k_cache, v_cache, table, layout=layout)
    desc.num_blocks = NB
    if stream is None:
        stream = torch.cuda.current_stream(k_cache.device).cuda_stream
    rc = lib.paged_attn_copy_blocks(ctypes.byref(desc), k_cache.data_ptr(), v_cache.data_ptr(),
                                    pairs.data_ptr(), pairs.shape[0],
                                    status.data_ptr() if status is not None else None, int(stream))
    if rc != 0:
        raise PagedAttnError(rc, "paged_attn_copy_blocks: ")
