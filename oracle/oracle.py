"""ctypes binding of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
CPU-baseline leg are the only callers. It imports nothing from the GPU package
and takes plain numpy arrays.

The oracle computes, for each sequence b and query head h, the full softmax of
``scale * Q[b,h] . K[t]`` over the L_b cached tokens, applied to V, gathering
token t from block ``block_table[b, t // bs]`` at offset ``t % bs`` and reading KV
head ``h // (H_q / H_kv)`` (page "Paged Attention Kernel Architecture for
BI-V100", sections 1, 3 and 4; decode-path example of the paged-attention docs
page). ``paged_attn_prefill`` is the varlen (many queries per sequence, causal)
form over the same paged pool (varlen path of that docs page). See
``oracle.c`` for the arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ERRORS = {0: "ok", -1: "bad argument", -2: "table entry out of range", -3: "bad cache length",
          -4: "out of memory"}

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (plain C, fp64, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.environ.get("ORACLE_LIB") and (
            not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH)):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    p = ctypes.c_void_p
    i = ctypes.c_int
    lib.oracle_paged_attn_pairs.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, p,
                                            ctypes.c_double, p, i, p, i]
    lib.oracle_paged_attn_pairs.restype = i
    lib.oracle_paged_prefill_pairs.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p, i,
                                               ctypes.c_double, p, i, p]
    lib.oracle_paged_prefill_pairs.restype = i
    lib.oracle_token_slot.argtypes = [p, i, i, i, i, i, p, p]
    lib.oracle_token_slot.restype = i
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def default_threads() -> int:
    """Worker threads when the caller names none: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def pool_strides(layout: str, Hkv: int, bs: int, D: int) -> tuple[int, int, int]:
    """(block, head, token) strides in elements for the two supported pool layouts."""
    if layout == "HND":  # [NB, H_kv, bs, D]
        return (Hkv * bs * D, bs * D, D)
    if layout == "NHD":  # [NB, bs, H_kv, D]
        return (bs * Hkv * D, D, Hkv * D)
    raise ValueError(layout)


def paged_attn_decode(q, k_pool, v_pool, block_table, seqlens, scale, *, kv_dtype, block_size,
                      num_kv_heads, layout="HND", pairs=None, nthreads=None):
    """fp64 attention outputs.

    ``k_pool``/``v_pool`` start at physical block 0 (any guard block in front of
    them is never touched unless a table entry is negative, which is an error).
    Returns ``[B, H_q, D]`` float64, or ``[len(pairs), D]`` when ``pairs`` (an
    ``[n, 2]`` array of (b, h)) is given.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    seql = np.ascontiguousarray(seqlens, dtype=np.int32)
    MBS = table.shape[1]
    assert table.shape[0] == B and seql.shape == (B,)
    NB = k_pool.shape[0]
    want = np.float32 if kv_dtype == "f32" else np.uint16
    assert k_pool.dtype == want and v_pool.dtype == want
    ks = np.array(pool_strides(layout, num_kv_heads, block_size, D), dtype=np.int64)
    for arr in (k_pool, v_pool):
        st = tuple(s // arr.itemsize for s in arr.strides)
        exp_shape = (NB, num_kv_heads, block_size, D) if layout == "HND" else (NB, block_size, num_kv_heads, D)
        assert arr.shape == exp_shape, (arr.shape, exp_shape)
        assert st[-1] == 1 and st[0] == ks[0], "pool must be a dense array"
    full = pairs is None
    if full:
        bb, hh = np.meshgrid(np.arange(B), np.arange(Hq), indexing="ij")
        pairs = np.stack([bb.ravel(), hh.ravel()], axis=1)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    out = np.zeros((pairs.shape[0], D), dtype=np.float64)
    if nthreads is None:
        nthreads = default_threads()
    rc = lib.oracle_paged_attn_pairs(
        B, Hq, num_kv_heads, D, block_size, NB, MBS, _DTYPE_CODE[kv_dtype],
        q.ctypes.data, k_pool.ctypes.data, v_pool.ctypes.data, ks.ctypes.data, ks.ctypes.data,
        table.ctypes.data, seql.ctypes.data, float(np.float32(scale)), pairs.ctypes.data,
        pairs.shape[0], out.ctypes.data, int(nthreads))
    if rc != 0:
        raise OracleError(f"oracle: {ERRORS.get(rc, rc)}")
    return out.reshape(B, Hq, D) if full else out


def paged_attn_prefill(q, k_pool, v_pool, block_table, cu_seqlens_q, seqlens_k, scale, *, causal,
                       kv_dtype, block_size, num_kv_heads, layout="HND", pairs=None,
                       nthreads=None):
    """fp64 outputs of the paged varlen prefill.

    ``q`` is ``[total_q, H_q, D]``; rows ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1``
    are sequence b's queries (the varlen indexing of the paged-attention docs
    page, varlen path), its keys the ``seqlens_k[b]`` tokens its table maps
    (the new ones included). With ``causal`` row i of a sequence with q_len
    queries and L keys attends tokens ``[0, L - q_len + i]`` (none when that is
    negative, giving zeros), else all L. Returns ``[total_q, H_q, D]`` float64,
    or ``[len(pairs), D]`` for an ``[n, 2]`` array of (row, h). The pairs are
    split into ``nthreads`` contiguous slices, each computed by its own call
    into the C function on a worker thread (the calls release the GIL); the
    arithmetic of every pair is the same whatever the split.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    total_q, Hq, D = q.shape
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    sk = np.ascontiguousarray(seqlens_k, dtype=np.int32)
    B, MBS = table.shape
    assert cu.shape == (B + 1,) and sk.shape == (B,) and int(cu[-1]) == total_q
    NB = k_pool.shape[0]
    want = np.float32 if kv_dtype == "f32" else np.uint16
    assert k_pool.dtype == want and v_pool.dtype == want
    ks = np.array(pool_strides(layout, num_kv_heads, block_size, D), dtype=np.int64)
    for arr in (k_pool, v_pool):
        st = tuple(s // arr.itemsize for s in arr.strides)
        assert st[-1] == 1 and st[0] == ks[0], "pool must be a dense array"
    full = pairs is None
    if full:
        rr, hh = np.meshgrid(np.arange(total_q), np.arange(Hq), indexing="ij")
        pairs = np.stack([rr.ravel(), hh.ravel()], axis=1)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    out = np.zeros((pairs.shape[0], D), dtype=np.float64)
    n = pairs.shape[0]
    if nthreads is None:
        nthreads = default_threads()
    nthreads = max(1, min(int(nthreads), n))

    def run(lo, hi):
        return lib.oracle_paged_prefill_pairs(
            B, Hq, num_kv_heads, D, block_size, NB, MBS, _DTYPE_CODE[kv_dtype],
            q.ctypes.data, k_pool.ctypes.data, v_pool.ctypes.data, ks.ctypes.data, ks.ctypes.data,
            table.ctypes.data, cu.ctypes.data, sk.ctypes.data, int(bool(causal)),
            float(np.float32(scale)), pairs[lo:hi].ctypes.data, hi - lo, out[lo:hi].ctypes.data)

    cuts = [n * i // nthreads for i in range(nthreads + 1)]
    if nthreads == 1:
        codes = [run(0, n)]
    else:
        import concurrent.futures as cf

        with cf.ThreadPoolExecutor(nthreads) as ex:
            codes = list(ex.map(run, cuts[:-1], cuts[1:]))
    rc = next((c for c in codes if c != 0), 0)
    if rc != 0:
        raise OracleError(f"oracle: {ERRORS.get(rc, rc)}")
    return out.reshape(total_q, Hq, D) if full else out


def token_slot(block_table, block_size, num_blocks, b, t):
    """(physical block, offset) that token t of sequence b is read from."""
    lib = _load()
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    ph = ctypes.c_int32()
    off = ctypes.c_int32()
    rc = lib.oracle_token_slot(table.ctypes.data, table.shape[1], block_size, num_blocks, b, t,
                               ctypes.byref(ph), ctypes.byref(off))
    return ph.value, off.value, rc


def decode16(bits, kv_dtype):
    """The oracle's own fp16 / bf16 decoders, elementwise (for pinning them)."""
    lib = _load()
    f = lib.oracle_decode_f16 if kv_dtype == "f16" else lib.oracle_decode_bf16
    return np.array([f(int(x)) for x in np.asarray(bits, dtype=np.uint16).ravel()], dtype=np.float64)
