"""Paged GQA decode attention for MI355X (gfx950).

``paged_attn_decode`` computes, for every sequence b and query head h, the
softmax-weighted sum of V over the ``cache_seqlens[b]`` tokens the block table
maps into a paged K/V pool, with G = H_q / H_kv query heads sharing each KV head.
The work runs in the HIP kernels of ``libpagedattn.so`` (C ABI in
``include/paged_attn.h``); this package only marshals torch tensors into that
call. Build the library with ``python -m paged_gqa_decode_block_amd.build``.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, PA_DTYPE, PA_FLAG_KV_SHARED, PA_FLAG_KV_XPACKED, PA_FLAG_QO_BF16, PA_PATH, PA_STATUS_BAD_BLOCK,
    PA_STATIC_SCRATCH_BYTES, PA_STATUS_BAD_SEQLEN, PATH_NAME,
    PaDesc, PagedAttnError, check_inputs, decode_append_raw, decode_raw, decode_static_raw,
    load_library, make_desc,
    partition_size, prefill_raw, prefill_workspace_size, prefill_workspace_zeroed_bytes,
    resolved_path, strerror, validate, workspace_size,
)

from .block_manager import BlockManager, copy_blocks  # noqa: E402,F401

_TORCH_DTYPE_NAME = {"torch.float32": "f32", "torch.float16": "f16", "torch.bfloat16": "bf16"}
_ws_cache: dict = {}
_ws_zero: dict = {}  # merged-grid workspaces: leading bytes known to be zero
_ws_retired: list = []  # outgrown workspaces, kept alive for graphs captured with them


def _kv_dtype(t) -> str:
    name = str(t.dtype)
    if name not in _TORCH_DTYPE_NAME:
        raise TypeError(f"K/V dtype {t.dtype} is not float32, float16 or bfloat16")
    return _TORCH_DTYPE_NAME[name]


def desc_for(q, k_cache, v_cache, block_table, *, layout="HND", partition_size=0, path="auto",
             kv_shared=False):
    """Descriptor for torch tensors. ``k_cache``/``v_cache`` are [NB, H_kv, bs, d]
    ("HND") or [NB, bs, H_kv, d] ("NHD"), any strides with d contiguous; or
    "XPACKED": K [NB, H_kv, d/x, bs, x] with x = 16 bytes / element and V
    [NB, H_kv, d, bs], dense within each (block, head) tile.
    ``kv_shared`` says physical blocks may be listed by several sequences."""
    B, Hq, D = q.shape
    if layout == "XPACKED":
        NB, Hkv, dx, bs, x = k_cache.shape
        if x * k_cache.element_size() != 16 or dx * x != D:
            raise ValueError("x-packed k_cache must be [NB, H_kv, d/x, bs, x], x = 16 bytes / element")
        if tuple(v_cache.shape) != (NB, Hkv, D, bs):
            raise ValueError("x-packed v_cache must be [NB, H_kv, d, bs]")
        if (k_cache.stride(4), k_cache.stride(3), k_cache.stride(2)) != (1, x, bs * x) or \
                (v_cache.stride(3), v_cache.stride(2)) != (1, bs):
            raise ValueError("x-packed K/V tiles must be dense within each (block, head)")
        return make_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                         num_blocks=NB, max_blocks_per_seq=block_table.shape[1],
                         kv_dtype=_kv_dtype(k_cache),
                         k_strides=(k_cache.stride(0), k_cache.stride(1), x),
                         v_strides=(v_cache.stride(0), v_cache.stride(1), 1),
                         partition_size=partition_size, path=path, kv_shared=kv_shared,
                         qo_bf16=str(q.dtype) == "torch.bfloat16", xpacked=True)
    if layout == "HND":
        NB, Hkv, bs, D2 = k_cache.shape
        ks = (k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))
        vs = (v_cache.stride(0), v_cache.stride(1), v_cache.stride(2))
    elif layout == "NHD":
        NB, bs, Hkv, D2 = k_cache.shape
        ks = (k_cache.stride(0), k_cache.stride(2), k_cache.stride(1))
        vs = (v_cache.stride(0), v_cache.stride(2), v_cache.stride(1))
    else:
        raise ValueError(f"layout must be 'HND', 'NHD' or 'XPACKED', got {layout!r}")
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q, k_cache and v_cache disagree on shape")
    if k_cache.stride(3) != 1 or v_cache.stride(3) != 1:
        raise ValueError("head_dim must be the contiguous axis of k_cache and v_cache")
    return make_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                     num_blocks=NB, max_blocks_per_seq=block_table.shape[1],
                     kv_dtype=_kv_dtype(k_cache), k_strides=ks, v_strides=vs,
                     partition_size=partition_size, path=path, kv_shared=kv_shared,
                     qo_bf16=str(q.dtype) == "torch.bfloat16")


def _check_q_tables(torch, q, block_table, cache_seqlens):
    if q.dtype not in (torch.float32, torch.bfloat16) or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 or bfloat16 tensor")
    for name, t in (("block_table", block_table), ("cache_seqlens", cache_seqlens)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")


def _check_out(q, out):
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")


def _on_stream(torch, stream, device):
    """Context in which torch enqueues on the raw stream handle ``stream``."""
    import contextlib

    if int(stream) == torch.cuda.current_stream(device).cuda_stream:
        return contextlib.nullcontext()
    return torch.cuda.stream(torch.cuda.ExternalStream(int(stream), device=device))


def workspace_for(desc: PaDesc, device, stream=None):
    """A cached device workspace of at least workspace_size(desc) bytes for calls
    enqueued on ``stream`` (a raw stream handle; torch's current stream when
    None).

    One workspace is kept per (device, stream, merged-grid or not): calls on one
    stream are ordered, so they may share it; calls on different streams get
    different ones. A workspace that a later call outgrows is replaced but never
    freed, because a HIP graph captured with it keeps its address and may still
    be replayed. The merged-grid path (``mfma_fused``) gets a workspace whose
    leading batch * num_kv_heads int32 arrival counters are zero: allocated
    zeroed, and zeroed again, on the launch stream, when a call needs more
    counters than the calls before it left zero (each call leaves its own
    counters zero)."""
    import torch

    n = workspace_size(desc)
    if n == 0:
        return None
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    fused = resolved_path(desc) == PA_PATH["mfma_fused"]
    key = (str(device), int(stream), fused)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < n:
        if ws is not None:
            _ws_retired.append(ws)
        with _on_stream(torch, stream, device):
            ws = (torch.zeros if fused else torch.empty)(n, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
        _ws_zero[key] = ws.numel() if fused else 0
    if fused:
        cnt_bytes = 4 * desc.batch * desc.num_kv_heads
        if cnt_bytes > _ws_zero[key]:
            with _on_stream(torch, stream, device):
                ws[:cnt_bytes].zero_()
        _ws_zero[key] = cnt_bytes
    return ws


_pf_ws_cache: dict = {}


def prefill_workspace_for(desc: PaDesc, max_seqlen_q: int, device, stream=None):
    """A cached device workspace for paged_attn_prefill's key split (None when
    the launch splits nothing), for calls enqueued on ``stream``.

    One workspace per (device, stream), allocated zeroed: its leading arrival
    counters must be zero when a call starts, and every call leaves them zero.
    A workspace that a later call outgrows is replaced but never freed (a HIP
    graph captured with it keeps its address)."""
    import torch

    n = prefill_workspace_size(desc, max_seqlen_q)
    if n == 0:
        return None
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    key = (str(device), int(stream))
    ws = _pf_ws_cache.get(key)
    if ws is None or ws.numel() < n:
        if ws is not None:
            _ws_retired.append(ws)
        with _on_stream(torch, stream, device):
            ws = torch.zeros(n, dtype=torch.uint8, device=device)
        _pf_ws_cache[key] = ws
    return ws


def paged_attn_decode(q, k_cache, v_cache, block_table, cache_seqlens, scale, out=None, *,
                      layout="HND", partition_size=0, path="auto", workspace=None, status=None,
                      stream=None, phase="both", kv_shared=False):
    """Single-query paged GQA attention; returns ``out`` ([B, H_q, d], q's dtype).

    q float32 or bfloat16 [B, H_q, d] (out has the same dtype; accumulation is
    fp32 either way); block_table int32 [B, MBS]; cache_seqlens int32 [B];
    all on one GPU. Enqueued on ``stream`` (default: torch's current stream).
    ``status`` is an optional int32 device tensor the kernels OR error bits into.
    ``phase`` "partition" or "combine" runs one of the two kernels alone (the
    combine phase needs the workspace the partition phase filled).
    ``kv_shared``: blocks may be listed by several sequences (prefix sharing);
    K/V then stay cacheable instead of being streamed non-temporally.
    """
    import torch

    if not q.is_cuda:
        raise ValueError("paged_attn_decode runs on the GPU; q is on the CPU")
    _check_q_tables(torch, q, block_table, cache_seqlens)
    desc = desc_for(q, k_cache, v_cache, block_table, layout=layout,
                    partition_size=partition_size, path=path, kv_shared=kv_shared)
    if out is None:
        out = torch.empty_like(q)
    _check_out(q, out)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None:
        workspace = workspace_for(desc, q.device, stream)
    rc = decode_raw(
        desc, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        cache_seqlens.data_ptr(), float(scale), out.data_ptr(),
        workspace.data_ptr() if workspace is not None else 0,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        status.data_ptr() if status is not None else 0, int(stream), phase)
    if rc != 0:
        raise PagedAttnError(rc, "paged_attn_decode: ")
    return out


def paged_attn_decode_static(q, k_cache, v_cache, block_table, cache_seqlens, scale, out, *,
                             layout="HND", partition_size=0, path="auto", status=None, stream=None,
                             kv_shared=False):
    """``paged_attn_decode`` on the library's static scratch instead of a
    workspace (paged_attn_decode_static in the C ABI): allocates nothing, so
    ``out`` must be given. Raises PagedAttnError with PA_E_SCRATCH when the call
    would need more than PA_STATIC_SCRATCH_BYTES of workspace. Calls that may
    overlap in time on one GPU share the scratch and race; keep them on one
    stream."""
    import torch

    if not q.is_cuda:
        raise ValueError("paged_attn_decode_static runs on the GPU; q is on the CPU")
    _check_q_tables(torch, q, block_table, cache_seqlens)
    desc = desc_for(q, k_cache, v_cache, block_table, layout=layout,
                    partition_size=partition_size, path=path, kv_shared=kv_shared)
    _check_out(q, out)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = decode_static_raw(desc, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                           block_table.data_ptr(), cache_seqlens.data_ptr(), float(scale),
                           out.data_ptr(), status.data_ptr() if status is not None else 0,
                           int(stream))
    if rc != 0:
        raise PagedAttnError(rc, "paged_attn_decode_static: ")
    return out


def paged_attn_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, scale,
                             out=None, *, layout="HND", partition_size=0, path="auto",
                             workspace=None, status=None, stream=None, kv_shared=False):
    """The decode step with the new token: writes ``k_new``/``v_new`` ([B, H_kv, d],
    the cache's dtype) at token ``cache_seqlens[b]`` of each sequence's paged cache,
    then attends ``cache_seqlens[b] + 1`` tokens. ``cache_seqlens`` is not changed.
    No allocation happens when ``out`` and ``workspace`` are given (or the cached
    workspace already exists), so the call can be captured in a CUDA/HIP graph."""
    import torch

    if not q.is_cuda:
        raise ValueError("paged_attn_decode_append runs on the GPU; q is on the CPU")
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2] if layout == "NHD" else k_cache.shape[1]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dtype != k_cache.dtype or tuple(t.shape) != (B, Hkv, D) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H_kv, d] tensor of the cache's dtype")
    _check_q_tables(torch, q, block_table, cache_seqlens)
    desc = desc_for(q, k_cache, v_cache, block_table, layout=layout,
                    partition_size=partition_size, path=path, kv_shared=kv_shared)
    if out is None:
        out = torch.empty_like(q)
    _check_out(q, out)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None:
        workspace = workspace_for(desc, q.device, stream)
    rc = decode_append_raw(
        desc, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_table.data_ptr(), cache_seqlens.data_ptr(), float(scale),
        out.data_ptr(), workspace.data_ptr() if workspace is not None else 0,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        status.data_ptr() if status is not None else 0, int(stream))
    if rc != 0:
        raise PagedAttnError(rc, "paged_attn_decode_append: ")
    return out


def paged_attn_prefill(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, scale, out=None,
                       *, max_seqlen_q=None, causal=True, layout="HND", status=None, stream=None,
                       split=True):
    """Paged varlen prefill; returns ``out`` ([total_q, H_q, d], q's dtype).

    Sequence b owns query rows ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1`` of the
    packed ``q`` ([total_q, H_q, d], float32 or bfloat16) and attends the
    ``seqlens_k[b]`` tokens its ``block_table`` row maps (the new ones included).
    With ``causal`` row i of a sequence with q_len rows and L keys attends tokens
    ``[0, L - q_len + i]`` (zeros when none), else all L. ``max_seqlen_q`` must
    bound every q_len; when None it is read from ``cu_seqlens_q`` (a device
    synchronisation, so pass it for graph capture). K/V must be float16 or
    bfloat16. ``split``: give the launch its key-split workspace (cached per
    device and stream, see prefill_workspace_for); False runs every work item
    whole.
    """
    import torch

    if not q.is_cuda:
        raise ValueError("paged_attn_prefill runs on the GPU; q is on the CPU")
    if q.dim() != 3:
        raise ValueError("q must be [total_q, H_q, d]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqlens_k", seqlens_k),
                    ("block_table", block_table)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    if q.dtype not in (torch.float32, torch.bfloat16) or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 or bfloat16 tensor")
    B = block_table.shape[0]
    if tuple(cu_seqlens_q.shape) != (B + 1,) or tuple(seqlens_k.shape) != (B,):
        raise ValueError("cu_seqlens_q must be [B + 1] and seqlens_k [B] for a [B, MBS] block_table")
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B > 0 else 0
    # the descriptor's batch is the number of sequences (q's first axis is rows)
    desc = desc_for(q, k_cache, v_cache, block_table, layout=layout)
    desc.batch = B
    if out is None:
        out = torch.empty_like(q)
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    ws = prefill_workspace_for(desc, int(max_seqlen_q), q.device, int(stream)) if split else None
    rc = prefill_raw(desc, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                     block_table.data_ptr(), cu_seqlens_q.data_ptr(), seqlens_k.data_ptr(),
                     int(max_seqlen_q), bool(causal), float(scale), out.data_ptr(),
                     ws.data_ptr() if ws is not None else 0, ws.numel() if ws is not None else 0,
                     status.data_ptr() if status is not None else 0, int(stream))
    if rc != 0:
        raise PagedAttnError(rc, "paged_attn_prefill: ")
    return out
