"""ctypes binding of libpagedattn.so (the C ABI in include/paged_attn.h).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. If the library
is not built this module raises on first use; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedattn.so")

PA_DTYPE = {"f32": 0, "f16": 1, "bf16": 2}
PA_PATH = {"auto": 0, "valu": 1, "mfma": 2, "mfma_grid": 3, "mfma_stream": 4, "mfma_fused": 5}
PATH_NAME = {1: "valu", 3: "mfma_grid", 4: "mfma_stream", 5: "mfma_fused"}

PA_OK = 0
PA_E = {
    -1: "PA_E_NULL", -2: "PA_E_SHAPE", -3: "PA_E_HEAD_DIM", -4: "PA_E_BLOCK_SIZE",
    -5: "PA_E_DTYPE", -6: "PA_E_STRIDE", -7: "PA_E_ALIGN", -8: "PA_E_PARTITION",
    -9: "PA_E_WORKSPACE", -10: "PA_E_PATH", -11: "PA_E_LAUNCH", -12: "PA_E_TABLE",
    -13: "PA_E_SEQLEN", -14: "PA_E_NOMEM", -15: "PA_E_SEQ", -16: "PA_E_SCRATCH",
}
PA_STATIC_SCRATCH_BYTES = 32 << 20
PA_FLAG_KV_SHARED = 1
PA_FLAG_QO_BF16 = 2
PA_FLAG_KV_XPACKED = 4
PA_STATUS_BAD_BLOCK = 1
PA_STATUS_BAD_SEQLEN = 2

EXPORTED = (
    "paged_attn_decode", "paged_attn_decode_static", "paged_attn_decode_append",
    "paged_attn_partition_phase",
    "paged_attn_combine_phase", "paged_attn_prefill", "paged_attn_prefill_workspace_size",
    "paged_attn_prefill_workspace_zeroed_bytes",
    "paged_attn_workspace_size", "paged_attn_validate", "paged_attn_partition_size", "paged_attn_resolved_path", "paged_attn_check_inputs",
    "paged_attn_strerror", "paged_attn_abi_version",
    # include/paged_block_manager.h
    "paged_attn_bm_create", "paged_attn_bm_destroy", "paged_attn_bm_allocate_blocks",
    "paged_attn_bm_free_sequence", "paged_attn_bm_share_prefix", "paged_attn_bm_cow_block",
    "paged_attn_bm_append_slot", "paged_attn_bm_num_free", "paged_attn_bm_ref_count",
    "paged_attn_bm_sequence_blocks", "paged_attn_bm_block_table", "paged_attn_copy_blocks",
)


class PaDesc(ctypes.Structure):
    """Mirror of ``pa_desc``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_stride_block", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("k_stride_token", ctypes.c_int64),
        ("v_stride_block", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64),
        ("partition_size", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        self.code = code
        super().__init__(f"{where}{PA_E.get(code, code)}: {strerror(code)}")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpagedattn.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_gqa_decode_block_amd.build` "
            "(hipcc, --offload-arch=gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dp = ctypes.POINTER(PaDesc)
    lib.paged_attn_decode.argtypes = [dp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, sz, vp, vp]
    lib.paged_attn_decode.restype = i32
    lib.paged_attn_decode_static.argtypes = [dp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.paged_attn_decode_static.restype = i32
    lib.paged_attn_decode_append.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                             sz, vp, vp]
    lib.paged_attn_decode_append.restype = i32
    lib.paged_attn_partition_phase.argtypes = lib.paged_attn_decode.argtypes
    lib.paged_attn_partition_phase.restype = i32
    lib.paged_attn_combine_phase.argtypes = [dp, vp, vp, vp, sz, vp]
    lib.paged_attn_combine_phase.restype = i32
    lib.paged_attn_prefill.argtypes = [dp, vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp,
                                       sz, vp, vp]
    lib.paged_attn_prefill.restype = i32
    lib.paged_attn_prefill_workspace_size.argtypes = [dp, i32]
    lib.paged_attn_prefill_workspace_size.restype = sz
    lib.paged_attn_prefill_workspace_zeroed_bytes.argtypes = [dp, i32]
    lib.paged_attn_prefill_workspace_zeroed_bytes.restype = sz
    lib.paged_attn_workspace_size.argtypes = [dp]
    lib.paged_attn_workspace_size.restype = sz
    lib.paged_attn_validate.argtypes = [dp]
    lib.paged_attn_validate.restype = i32
    lib.paged_attn_partition_size.argtypes = [dp]
    lib.paged_attn_partition_size.restype = i32
    lib.paged_attn_resolved_path.argtypes = [dp]
    lib.paged_attn_resolved_path.restype = i32
    lib.paged_attn_check_inputs.argtypes = [dp, vp, vp]
    lib.paged_attn_check_inputs.restype = i32
    lib.paged_attn_strerror.argtypes = [i32]
    lib.paged_attn_strerror.restype = ctypes.c_char_p
    lib.paged_attn_abi_version.argtypes = []
    lib.paged_attn_abi_version.restype = i32
    i64, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
    lib.paged_attn_bm_create.argtypes = [i32, i32]
    lib.paged_attn_bm_create.restype = vp
    lib.paged_attn_bm_destroy.argtypes = [vp]
    lib.paged_attn_bm_destroy.restype = None
    lib.paged_attn_bm_allocate_blocks.argtypes = [vp, i64, i32]
    lib.paged_attn_bm_free_sequence.argtypes = [vp, i64]
    lib.paged_attn_bm_share_prefix.argtypes = [vp, i64, i64, i32]
    lib.paged_attn_bm_cow_block.argtypes = [vp, i64, i32, ip, ip]
    lib.paged_attn_bm_append_slot.argtypes = [vp, i64, i32, ip, ip]
    lib.paged_attn_bm_num_free.argtypes = [vp]
    lib.paged_attn_bm_ref_count.argtypes = [vp, i32]
    lib.paged_attn_bm_sequence_blocks.argtypes = [vp, i64, ip, i32]
    lib.paged_attn_bm_block_table.argtypes = [vp, ctypes.POINTER(ctypes.c_int64), i32, i32, ip]
    lib.paged_attn_copy_blocks.argtypes = [dp, vp, vp, vp, i32, vp, vp]
    for name in ("paged_attn_bm_allocate_blocks", "paged_attn_bm_free_sequence",
                 "paged_attn_bm_share_prefix", "paged_attn_bm_cow_block", "paged_attn_bm_append_slot",
                 "paged_attn_bm_num_free", "paged_attn_bm_ref_count", "paged_attn_bm_sequence_blocks",
                 "paged_attn_bm_block_table", "paged_attn_copy_blocks"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().paged_attn_strerror(int(code)).decode()


def make_desc(*, batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
              max_blocks_per_seq, kv_dtype, k_strides, v_strides=None, partition_size=0,
              path="auto", kv_shared=False, qo_bf16=False, xpacked=False) -> PaDesc:
    v_strides = k_strides if v_strides is None else v_strides
    return PaDesc(
        int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(num_blocks), int(max_blocks_per_seq),
        PA_DTYPE[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype),
        *[int(x) for x in k_strides], *[int(x) for x in v_strides], int(partition_size),
        PA_PATH[path] if isinstance(path, str) else int(path),
        (PA_FLAG_KV_SHARED if kv_shared else 0) | (PA_FLAG_QO_BF16 if qo_bf16 else 0)
        | (PA_FLAG_KV_XPACKED if xpacked else 0), 0)


def validate(desc: PaDesc) -> int:
    return load_library().paged_attn_validate(ctypes.byref(desc))


def workspace_size(desc: PaDesc) -> int:
    return int(load_library().paged_attn_workspace_size(ctypes.byref(desc)))


def prefill_workspace_size(desc: PaDesc, max_seqlen_q: int) -> int:
    """Bytes of the prefill's key-split workspace (0: no work item is split)."""
    return int(load_library().paged_attn_prefill_workspace_size(ctypes.byref(desc),
                                                                int(max_seqlen_q)))


def prefill_workspace_zeroed_bytes(desc: PaDesc, max_seqlen_q: int) -> int:
    """Leading bytes of that workspace (arrival counters) that must be zero."""
    return int(load_library().paged_attn_prefill_workspace_zeroed_bytes(ctypes.byref(desc),
                                                                        int(max_seqlen_q)))


def decode_append_raw(desc: PaDesc, q_ptr: int, knew_ptr: int, vnew_ptr: int, k_ptr: int, v_ptr: int,
                      table_ptr: int, seqlens_ptr: int, scale: float, out_ptr: int, ws_ptr: int,
                      ws_bytes: int, status_ptr: int, stream: int) -> int:
    """Direct call of paged_attn_decode_append with integer device addresses."""
    return int(load_library().paged_attn_decode_append(
        ctypes.byref(desc), q_ptr, knew_ptr, vnew_ptr, k_ptr, v_ptr, table_ptr, seqlens_ptr,
        ctypes.c_float(scale), out_ptr, ws_ptr, ws_bytes, status_ptr, stream))


def partition_size(desc: PaDesc) -> int:
    return int(load_library().paged_attn_partition_size(ctypes.byref(desc)))


def resolved_path(desc: PaDesc) -> int:
    return int(load_library().paged_attn_resolved_path(ctypes.byref(desc)))


def check_inputs(desc: PaDesc, block_table_host, seqlens_host) -> int:
    """Host-side value check of numpy int32 copies of the table and lengths."""
    import numpy as np

    t = np.ascontiguousarray(block_table_host, dtype=np.int32)
    s = np.ascontiguousarray(seqlens_host, dtype=np.int32)
    return load_library().paged_attn_check_inputs(ctypes.byref(desc), t.ctypes.data, s.ctypes.data)


def prefill_raw(desc: PaDesc, q_ptr: int, k_ptr: int, v_ptr: int, table_ptr: int, cu_q_ptr: int,
                seqlens_k_ptr: int, max_seqlen_q: int, causal: bool, scale: float, out_ptr: int,
                ws_ptr: int, ws_bytes: int, status_ptr: int, stream: int) -> int:
    """Direct call of paged_attn_prefill with integer device addresses."""
    return int(load_library().paged_attn_prefill(
        ctypes.byref(desc), q_ptr or None, k_ptr or None, v_ptr or None, table_ptr or None,
        cu_q_ptr or None, seqlens_k_ptr or None, int(max_seqlen_q), int(bool(causal)),
        ctypes.c_float(scale), out_ptr or None, ws_ptr or None, int(ws_bytes), status_ptr or None,
        stream or None))


def decode_static_raw(desc: PaDesc, q_ptr: int, k_ptr: int, v_ptr: int, table_ptr: int,
                      seqlens_ptr: int, scale: float, out_ptr: int, status_ptr: int,
                      stream: int) -> int:
    """Direct call of paged_attn_decode_static (no workspace argument) with
    integer device addresses."""
    return int(load_library().paged_attn_decode_static(
        ctypes.byref(desc), q_ptr or None, k_ptr or None, v_ptr or None, table_ptr or None,
        seqlens_ptr or None, ctypes.c_float(scale), out_ptr or None, status_ptr or None,
        stream or None))


def decode_raw(desc: PaDesc, q_ptr: int, k_ptr: int, v_ptr: int, table_ptr: int, seqlens_ptr: int,
               scale: float, out_ptr: int, ws_ptr: int, ws_bytes: int, status_ptr: int,
               stream: int, phase: str = "both") -> int:
    """Direct call of paged_attn_decode (phase "both"), paged_attn_partition_phase
    ("partition") or paged_attn_combine_phase ("combine") with integer device
    addresses."""
    lib = load_library()
    if phase == "combine":
        return lib.paged_attn_combine_phase(ctypes.byref(desc), seqlens_ptr or None, out_ptr or None,
                                            ws_ptr or None, ws_bytes, stream or None)
    fn = lib.paged_attn_partition_phase if phase == "partition" else lib.paged_attn_decode
    return fn(
        ctypes.byref(desc), q_ptr or None, k_ptr or None, v_ptr or None, table_ptr or None,
        seqlens_ptr or None, ctypes.c_float(scale), out_ptr or None, ws_ptr or None, ws_bytes,
        status_ptr or None, stream or None)
