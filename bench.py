"""Decode-attention throughput on one MI355X: KV GB/s, % of HBM peak, seq-heads/s.

A step is one decode call (partition kernel + combine kernel) over the whole
synthetic batch, inputs resident in HBM. Default workload: the 64-sequence
large-GQA bf16 batch (B=64, H_q=64, H_kv=8, d=128, bs=16, lengths log-uniform in
[1024, 32768], 10% spare blocks); the 100K-token Qwen3.6-shaped batch (B=1,
H_q=24, H_kv=4, d=256, partition 512), the prefix-shared 256-sequence batch, and
(for information: they fit in the caches) the tiny fp32 example and the Qwen2-shaped
fp16 batch are measured too and reported under "also". Prints one JSON line on
stdout; progress goes to stderr.

Each step is timed two ways: flushed (a 1 GiB read evicts the L2s and the
256 MB MALL before every timed step, an event pair around the step alone; the
median of the K steps is ``ms_per_step`` and ``value``) and warm (K back-to-back
steps between one event pair, reported as ``warm_ms_per_step``). The CPU
baseline leg also compares the last timed step's whole output with the fp64
oracle (``max_abs_err``, ``parity``).

  python bench.py [--steps K] [--warmup W] [--config 4] [--also 3]
  python bench.py --profile partition   # only partition-kernel launches (for rocprofv3)
  python bench.py --profile copy        # a 1 GiB device copy (counter calibration)

Next to the decode numbers it reports plain HBM read rates on the same GPU
(libpaprobe.so: a 2 GiB buffer read sequentially and as 4 / 8 KB tiles in random
order) and the fp64 CPU oracle timed on a bounded sample (all threads and one).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8.0 TB/s
METRIC = "decode attention KV GB/s (% of MI355X HBM peak) + seq-heads/s, 1 GPU"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
# sources of the streaming partition kernel (the dominant one) and its launch:
# HBM counter readings taken on other sources are not reported as its traffic
KERNEL_SOURCES = ["paged_gqa_decode_block_amd/csrc/pa_partition_stream.hip",
                  "paged_gqa_decode_block_amd/csrc/pa_mfma_util.h",
                  "paged_gqa_decode_block_amd/csrc/pa_kernels.h",
                  "paged_gqa_decode_block_amd/csrc/pa_api.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Workload:
    """One generated configuration, copied to the GPU once."""

    def __init__(self, k: int, torch, path: str, partition: int | None = None,
                 layout: str = "HND", case=None, seed: int | None = None):
        from paged_gqa_decode_block_amd import workload as W
        import paged_gqa_decode_block_amd as pa

        if case is None:  # the tests hand in a case they generated already
            t = time.time()
            case = W.make_config(k)
            log(f"[bench] generated config {k} ({case.name}) in {time.time() - t:.1f}s")
        self.case = c = case
        self.k = k
        self.seed = 1000 + k if seed is None else seed
        self.torch = torch
        self.path = path

        def pool(store):
            if c.kv_dtype == "f32":
                x = torch.from_numpy(np.ascontiguousarray(store))
            else:
                x = torch.from_numpy(np.ascontiguousarray(store).view(np.int16)).view(
                    torch.bfloat16 if c.kv_dtype == "bf16" else torch.float16)
            return x.to("cuda")[1:]

        self.q = torch.from_numpy(c.q).to("cuda")
        if layout == "XPACKED":  # the same values, x-packed K / transposed V
            self.k_pool = pool(W.to_xpacked(c.k_store, "k"))
            self.v_pool = pool(W.to_xpacked(c.v_store, "v"))
        else:
            self.k_pool = pool(c.k_store)
            self.v_pool = pool(c.v_store)
        self.layout = layout if layout == "XPACKED" else c.layout
        self.table = torch.from_numpy(c.block_table).to("cuda")
        self.seqlens = torch.from_numpy(c.seqlens).to("cuda")
        self.out = torch.empty_like(self.q)
        # the prefix-shared workload's block manager knows blocks are listed by
        # several sequences (reference counts > 1): keep K/V loads cacheable
        self.kv_shared = c.ref_count is not None and int(c.ref_count.max()) > 1
        part = c.partition_size if k == 3 else 0  # the 100K-token workload fixes 512
        if partition is not None:
            part = partition
        self.desc = pa.desc_for(self.q, self.k_pool, self.v_pool, self.table, layout=self.layout,
                                partition_size=part, path=path, kv_shared=self.kv_shared)
        n = pa.workspace_size(self.desc)
        # zeroed: the merged grid variant keeps arrival counters (zero between
        # calls) at the start of its workspace
        self.ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
        self.part = pa.partition_size(self.desc)
        self.path_name = pa.PATH_NAME[pa.resolved_path(self.desc)]
        self.kv_bytes = c.kv_bytes()
        self.unique_kv_bytes = c.unique_kv_bytes() if c.ref_count is not None else self.kv_bytes
        self.stream = torch.cuda.current_stream()
        torch.cuda.synchronize()

    def call(self, phase="both", stream=None):
        import paged_gqa_decode_block_amd as pa

        st = self.stream.cuda_stream if stream is None else stream
        rc = pa.decode_raw(self.desc, self.q.data_ptr(), self.k_pool.data_ptr(),
                           self.v_pool.data_ptr(), self.table.data_ptr(), self.seqlens.data_ptr(),
                           self.case.scale, self.out.data_ptr(), self.ws.data_ptr(),
                           self.ws.numel(), 0, st, phase)
        if rc != 0:
            raise pa.PagedAttnError(rc, "bench: ")

    def describe(self) -> dict:
        c = self.case
        return {
            "workload": c.name, "batch": c.B, "num_q_heads": c.Hq, "num_kv_heads": c.Hkv,
            "head_dim": c.D, "block_size": c.bs, "kv_dtype": c.kv_dtype, "layout": self.layout,
            "partition_size": self.part, "path": self.path_name, "kv_shared": self.kv_shared,
            "total_cached_tokens": int(c.seqlens.astype(np.int64).sum()),
            "num_physical_blocks": c.NB, "seed": self.seed,
        }


def time_steps(torch, fn, steps: int) -> float:
    """ms per call of fn over `steps` back-to-back calls, HIP events on the launch stream."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_each(torch, fn, steps: int, flush=None) -> np.ndarray:
    """Per-call ms with an event pair around each call (optionally after a cache flush)."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def flush_caches(flush_buf):
    """Evict the decode's data from the L2s and the 256 MB MALL: read a 1 GiB
    buffer (a read, so no dirty lines are left to be written back during the
    next step)."""
    flush_buf.sum()


def measure(wl: Workload, steps: int, warmup: int, flush_buf) -> dict:
    """The step timed two ways: flushed (each step after a cache flush, its own
    event pair; the median is the headline) and warm (``steps`` back-to-back
    calls between one event pair)."""
    torch = wl.torch
    for _ in range(warmup):
        wl.call()
    cold_ms = time_each(torch, wl.call, steps, flush=lambda: flush_caches(flush_buf))
    ms = time_steps(torch, wl.call, steps)
    # the partition kernel alone: one event pair around `steps` back-to-back
    # launches on the launch stream (average launch duration), plus per-launch
    # event pairs for the spread
    part_avg_ms = time_steps(torch, lambda: wl.call("partition"), steps)
    part_ms = time_each(torch, lambda: wl.call("partition"), steps)
    wl.call()  # leave the workspace of a complete call behind for the combine timing
    comb_ms = time_steps(torch, lambda: wl.call("combine"), steps)
    step_each = time_each(torch, wl.call, steps)
    # the same step captured once in a HIP graph and replayed (the call
    # allocates nothing and never synchronises, so it captures as is)
    wl.call()
    torch.cuda.synchronize()
    eager_out = wl.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wl.call(stream=torch.cuda.current_stream().cuda_stream)
    same = True
    for _ in range(3):
        wl.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = same and bool(torch.equal(wl.out, eager_out))
    graph_ms = time_steps(torch, g.replay, steps)
    del g
    wl.call()
    torch.cuda.synchronize()
    c = wl.case
    cold = float(np.median(cold_ms))
    t = cold / 1e3
    return {
        "ms_per_step": cold,
        "kv_gbs": wl.kv_bytes / t / 1e9,
        "seq_heads_per_s": c.B * c.Hq / t,
        "cold_step_us_p10_p50_p90": [float(np.percentile(cold_ms, x) * 1e3) for x in (10, 50, 90)],
        "warm_ms_per_step": ms,
        "warm_kv_gbs": wl.kv_bytes / (ms / 1e3) / 1e9,
        "partition_kernel_us": float(part_avg_ms * 1e3),
        "partition_kernel_us_p10_p90": [float(np.percentile(part_ms, 10) * 1e3),
                                        float(np.percentile(part_ms, 90) * 1e3)],
        "combine_kernel_us": float(comb_ms * 1e3),
        "warm_step_us_p10_p50_p90": [float(np.percentile(step_each, x) * 1e3) for x in (10, 50, 90)],
        "graph_step_us": float(graph_ms * 1e3),
        "graph_output_equals_step": same,
        "kv_bytes": wl.kv_bytes,
        "unique_kv_bytes": wl.unique_kv_bytes,
        # prefix-shared blocks counted once (equal to kv_gbs when no block is shared)
        "unique_kv_gbs": wl.unique_kv_bytes / t / 1e9,
    }


def measure_brief(wl: Workload, steps: int, warmup: int, flush_buf) -> dict:
    """Flushed and warm step times and the partition kernel's average launch
    duration, for the context legs."""
    torch = wl.torch
    for _ in range(warmup):
        wl.call()
    cold = float(np.median(time_each(torch, wl.call, steps,
                                     flush=lambda: flush_caches(flush_buf))))
    warm = time_steps(torch, wl.call, steps)
    part = time_steps(torch, lambda: wl.call("partition"), steps)
    wl.call()
    torch.cuda.synchronize()
    return {"step_us": round(cold * 1e3, 2), "warm_step_us": round(warm * 1e3, 2),
            "partition_kernel_us": round(part * 1e3, 2),
            "kv_gbs": round(wl.kv_bytes / (cold / 1e3) / 1e9, 1),
            "partition_kernel_kv_gbs": round(wl.kv_bytes / (part / 1e3) / 1e9, 1),
            "kv_bytes": wl.kv_bytes, "path": wl.path_name, "partition_size": wl.part}


def gqa_sweep(wl: Workload, steps: int, warmup: int, flush_buf) -> dict:
    """The headline workload's K/V pool and tables with G = H_q / H_kv of 1, 2
    and 8 (the first 8, 16 and 64 query heads of each sequence): the K/V bytes
    a call must read do not depend on G (one pass over each KV head's tokens
    serves all G query heads of its group), so neither should the time."""
    from paged_gqa_decode_block_amd import workload as W

    c = wl.case
    out = {}
    for G in (1, 2, c.G):
        hq = G * c.Hkv
        cg = W.Case(**{**c.__dict__, "q": np.ascontiguousarray(c.q[:, :hq]), "Hq": hq,
                       "name": f"{c.name}_G{G}"})
        wg = Workload(4, wl.torch, wl.path, None, wl.layout, case=cg)
        out[f"G{G}"] = {"num_q_heads": hq, **measure_brief(wg, steps, warmup, flush_buf)}
        log(f"[bench] {c.name} with G = {G}: {out[f'G{G}']['step_us']:.1f} us/step flushed, "
            f"partition kernel {out[f'G{G}']['partition_kernel_us']:.1f} us")
        del wg
        wl.torch.cuda.empty_cache()
    return out


def shard_leg(torch, steps: int, warmup: int, flush_buf, n: int = 8) -> dict:
    """The 100K-token workload's context split by tokens over n GPUs: what one
    GPU computes (the partition kernel at one shard's real shape, 12 500
    tokens for n = 8, plus the merge of its own partitions). The exchange of
    the shards' partial states and their final merge are not part of it."""
    from paged_gqa_decode_block_amd import workload as W

    c = W.make_shard(n)
    r = {"shards": n}
    # the library's choice (one shard is a small batch), and the streaming
    # kernel at the whole workload's 512-token partitions
    for key, path, part in (("auto", "auto", 0), ("stream_512", "mfma_stream", 512)):
        wl = Workload(3, torch, path, part, case=c, seed=1003 + 100 * n)
        r[key] = {**wl.describe(), **measure_brief(wl, steps, warmup, flush_buf)}
        log(f"[bench] {c.name} ({key}): {r[key]['step_us']:.1f} us/step flushed, "
            f"{r[key]['kv_gbs']:.0f} GB/s")
        del wl
    torch.cuda.empty_cache()
    return r


# Throughput table of the paged-attention-runtime design notes (RTX 2070, SM75;
# Qwen2 shapes, head size 64, 14 query heads): concurrent sequences -> tokens/s.
RUNTIME_NOTES_RTX2070 = {1: 542981, 2: 844423, 4: 1239648, 8: 2890839}


def batch_sweep(torch, steps: int, warmup: int, flush_buf) -> dict:
    """Qwen2-shaped decode (H_q 14, H_kv 2, d 64, fp16 K/V, 512 cached tokens per
    sequence) for 1, 2, 4 and 8 sequences, and the speedup over one sequence,
    next to the design notes' RTX 2070 table for context (other hardware). The
    notes do not define their tokens/s; both readings are given: decode tokens
    (one query token per sequence per call) and cached tokens attended, each
    per second of call time."""
    from paged_gqa_decode_block_amd import workload as W

    out = {"context": {"source": "paged-attention-runtime design notes, throughput table",
                       "hardware": "RTX 2070 (SM75)", "tokens_per_s": RUNTIME_NOTES_RTX2070,
                       "speedup_8_over_1": round(RUNTIME_NOTES_RTX2070[8] / RUNTIME_NOTES_RTX2070[1], 2)}}
    base = None
    for B in (1, 2, 4, 8):
        c = W.make_qwen2_batch(B)
        wl = Workload(2, torch, "auto", None, case=c, seed=4000 + B)
        r = measure_brief(wl, steps, warmup, flush_buf)
        tps = B / (r["step_us"] / 1e6)
        tps_warm = B / (r["warm_step_us"] / 1e6)
        ctx_warm = int(c.seqlens.sum()) / (r["warm_step_us"] / 1e6)
        base = base or tps_warm
        out[f"B{B}"] = {**r, "tokens_per_s": round(tps, 1), "warm_tokens_per_s": round(tps_warm, 1),
                        "warm_cached_tokens_per_s": round(ctx_warm, 1),
                        "warm_speedup": round(tps_warm / base, 2)}
        log(f"[bench] {c.name}: {r['warm_step_us']:.1f} us/step warm, {tps_warm:.0f} tokens/s")
        del wl
    torch.cuda.empty_cache()
    return out


def measure_append_graph(wl: Workload, steps: int) -> dict:
    """The decode step with the new token (paged_attn_decode_append: append kernel,
    partition, combine), captured once in a HIP graph and replayed. Each replay
    appends every sequence's last cached token over itself (cache lengths minus
    one, K/V rows gathered from the cache) and attends the same L tokens, so the
    KV bytes and the output equal the plain step's."""
    import paged_gqa_decode_block_amd as pa

    torch = wl.torch
    c = wl.case
    L = wl.seqlens.long()
    Lm1 = (wl.seqlens - 1).clamp(min=0).contiguous()
    t = (L - 1).clamp(min=0)
    blk = wl.table.long().gather(1, (t // c.bs).unsqueeze(1)).squeeze(1).clamp(min=0)
    off = t % c.bs
    if wl.layout == "XPACKED":  # K [NB, H, d/8, bs, 8], V [NB, H, d, bs]
        kn = wl.k_pool[blk, :, :, off, :].reshape(c.B, c.Hkv, c.D)
        vn = wl.v_pool[blk, :, :, off]
    elif c.layout == "HND":
        kn, vn = wl.k_pool[blk, :, off, :], wl.v_pool[blk, :, off, :]
    else:
        kn, vn = wl.k_pool[blk, off, :, :], wl.v_pool[blk, off, :, :]
    kn, vn = kn.contiguous(), vn.contiguous()
    out = torch.empty_like(wl.q)

    def step():
        pa.paged_attn_decode_append(wl.q, kn, vn, wl.k_pool, wl.v_pool, wl.table, Lm1, c.scale, out,
                                    layout=wl.layout, partition_size=wl.part, path=wl.path,
                                    workspace=wl.ws, kv_shared=wl.kv_shared)

    step()
    wl.call()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, wl.out))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    ms = time_steps(torch, g.replay, steps)
    return {"append_graph_step_us": float(ms * 1e3),
            "append_graph_kv_gbs": wl.kv_bytes / (ms / 1e3) / 1e9,
            "append_output_equals_decode": same}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def measure_prefill(k: int, torch, steps: int, warmup: int) -> dict:
    """The paged varlen prefill (causal) on prefill workload k: one call per
    step, inputs resident on the GPU, q and out in bf16 (a bf16 model's
    prefill; the headline fields) and in fp32 (``fp32_q_out``). Useful flops
    count 2 multiply-adds per attended (query row, head, key, dim) for Q.K and
    the same for P.V. The matrix cores do exactly that work for bf16 q (Q and
    P each one 16-bit part); fp32 q goes in hi + lo parts, 1.5 times the
    work."""
    import paged_gqa_decode_block_amd as pa
    from paged_gqa_decode_block_amd import workload as W

    t = time.time()
    c, cu, q = W.make_prefill(k)
    log(f"[bench] generated prefill workload {k} ({c.name}) in {time.time() - t:.1f}s")

    def pool(store):
        return torch.from_numpy(np.ascontiguousarray(store).view(np.int16)).view(
            torch.bfloat16).to("cuda")[1:]

    qd = torch.from_numpy(q).to("cuda")
    qd16 = qd.to(torch.bfloat16)
    kp, vp = pool(c.k_store), pool(c.v_store)
    table = torch.from_numpy(c.block_table).to("cuda")
    cud = torch.from_numpy(cu).to("cuda")
    sk = torch.from_numpy(c.seqlens).to("cuda")
    out = torch.empty_like(qd)
    out16 = torch.empty_like(qd16)
    qlens = np.diff(cu).astype(np.int64)
    max_q = int(qlens.max())
    L = c.seqlens.astype(np.int64)
    keys = int((qlens * (L - qlens) + qlens * (qlens + 1) // 2).sum())   # attended (row, key) pairs
    flops = 4.0 * c.Hq * c.D * keys
    kv_bytes = int(L.sum()) * c.Hkv * c.D * 2 * 2

    def timed(qq, oo):
        def call():
            pa.paged_attn_prefill(qq, kp, vp, table, cud, sk, c.scale, oo, max_seqlen_q=max_q,
                                  causal=True)
        for _ in range(warmup):
            call()
        ms = time_steps(torch, call, steps)
        return ms, flops / (ms / 1e3) / 1e12

    ms, tf = timed(qd16, out16)
    ms32, tf32 = timed(qd, out)
    log(f"[bench] {c.name}: prefill {ms * 1e3:.1f} us/step, {tf:.1f} useful TFLOP/s (bf16 q/out); "
        f"{ms32 * 1e3:.1f} us/step, {tf32:.1f} TFLOP/s (fp32 q/out)")
    r = {"workload": c.name, "batch": c.B, "num_q_heads": c.Hq, "num_kv_heads": c.Hkv,
         "head_dim": c.D, "block_size": c.bs, "kv_dtype": c.kv_dtype, "q_out_dtype": "bf16",
         "causal": True, "total_q_rows": int(cu[-1]), "total_cached_tokens": int(L.sum()),
         "seed": 2000 + k, "us_per_step": round(ms * 1e3, 2), "useful_tflops": round(tf, 2),
         "kv_bytes": kv_bytes,
         "fp32_q_out": {"us_per_step": round(ms32 * 1e3, 2), "useful_tflops": round(tf32, 2),
                        "frac_of_bf16_peak": round(tf32 / MFMA_BF16_PEAK_TFLOPS, 4)},
         "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                      "traffic": None, "kernel": "prefill_kernel",
                      "algorithmic_flops_per_launch": flops}}
    del qd, qd16, kp, vp, out, out16
    torch.cuda.empty_cache()
    return r


def roofline(wl: Workload, r: dict) -> dict:
    """The partition kernel against the HBM peak. Algorithmic bytes: K and V
    of every distinct cached block once (the logical bytes unless blocks are
    listed by several sequences, as in the prefix-shared batch, where a kernel
    that reads a shared block once per listing moves more than it must)."""
    alg = wl.unique_kv_bytes
    achieved = alg / (r["partition_kernel_us"] / 1e6) / 1e9
    out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
           "kernel": f"partition_{wl.path_name}", "algorithmic_bytes_per_launch": alg}
    if alg != wl.kv_bytes:
        out["logical_bytes_per_launch"] = wl.kv_bytes
    try:
        with open(COUNTERS_FILE) as f:
            cnt = json.load(f)
        entry = cnt.get(wl.case.name, {})
        if entry.get("kernel_hash") == kernel_hash() and entry.get("path") == wl.path_name:
            hbm = entry["hbm_bytes_per_launch"]
            out["traffic"] = round(hbm / (r["partition_kernel_us"] / 1e6) / 1e9, 1)
            out["traffic_bytes_per_launch"] = hbm
    except (OSError, ValueError, KeyError):
        pass
    return out


def read_probe(torch, steps: int = 10) -> dict:
    """Plain HBM read rates on the same GPU, for context next to the decode
    kernel: a 2 GiB buffer read front to back, and the same buffer read as 4 KB
    and 8 KB tiles in a seeded random order (the K tile of one (block, KV head)
    at head_dim 128 and 256) by one-wave workgroups with three tiles in flight
    each, the decode kernel's shape; 16-byte non-temporal loads
    (libpaprobe.so)."""
    import ctypes

    from paged_gqa_decode_block_amd import build as B

    if not os.path.exists(B.PROBE_LIB):
        raise RuntimeError(f"{B.PROBE_LIB} is missing: build it with python -m "
                           "paged_gqa_decode_block_amd.build")
    lib = ctypes.CDLL(B.PROBE_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.pa_probe_stream_read.argtypes = [vp, i64, vp, i32, vp]
    lib.pa_probe_tile_gather.argtypes = [vp, vp, i32, i32, vp, i32, vp]
    nbytes = 1 << 31
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * cus
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4 * blocks, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    out = {"buffer_bytes": nbytes, "loads": "16-byte non-temporal",
           "sequential": f"{blocks} workgroups of 256 threads",
           "tiles": f"{blocks} one-wave workgroups, three tiles in flight per wave"}

    def timed(fn) -> float:
        for _ in range(3):
            fn()
        ms = time_steps(torch, fn, steps)
        return nbytes / (ms / 1e3) / 1e9

    def run(rc):
        if rc != 0:
            raise RuntimeError(f"read probe launch failed ({rc})")

    out["stream_read_gbs"] = round(timed(lambda: run(lib.pa_probe_stream_read(
        buf.data_ptr(), nbytes, sink.data_ptr(), blocks, st.cuda_stream))), 1)
    rng = np.random.default_rng(7)
    for kb in (4, 8):
        ntiles = nbytes // (kb * 1024)
        tiles = torch.from_numpy(rng.permutation(ntiles).astype(np.int32)).to("cuda")
        out[f"tile_gather_{kb}k_gbs"] = round(timed(lambda: run(lib.pa_probe_tile_gather(
            buf.data_ptr(), tiles.data_ptr(), ntiles, kb * 1024, sink.data_ptr(), blocks,
            st.cuda_stream))), 1)
        if kb == 8:
            # one read of as many bytes as the 100K-token decode moves (409.6 MB,
            # 50000 random 8 KB tiles): the bare gather's time for that size,
            # start-up and tail included
            n3 = 409_600_000 // 8192
            for _ in range(3):
                run(lib.pa_probe_tile_gather(buf.data_ptr(), tiles.data_ptr(), n3, 8192,
                                             sink.data_ptr(), blocks, st.cuda_stream))
            ms3 = time_steps(torch, lambda: run(lib.pa_probe_tile_gather(
                buf.data_ptr(), tiles.data_ptr(), n3, 8192, sink.data_ptr(), blocks,
                st.cuda_stream)), steps)
            out["tile_gather_8k_409mb_us"] = round(ms3 * 1e3, 2)
            out["tile_gather_8k_409mb_gbs"] = round(n3 * 8192 / (ms3 / 1e3) / 1e9, 1)
        del tiles
    del buf, sink
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PARITY_TOL = {"f32": 1e-5, "f16": 3e-3, "bf16": 3e-3}


def cpu_baseline_parity(wl: Workload, got: np.ndarray) -> dict:
    """Part of the CPU-baseline leg: the fp64 oracle over the whole batch of the
    workload, compared element by element with the output of the last timed
    step (``got``, [B, H_q, d] as floats). The tolerance is the one the GPU
    tests hold: 1e-5 for fp32 K/V, 3e-3 for 16-bit K/V."""
    from oracle import oracle as O

    c = wl.case
    t0 = time.perf_counter()
    want = O.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seqlens, c.scale,
                               kv_dtype=c.kv_dtype, block_size=c.bs, num_kv_heads=c.Hkv,
                               layout=c.layout)
    dt = time.perf_counter() - t0
    finite = bool(np.isfinite(got).all())
    err = float(np.abs(got.astype(np.float64) - want).max()) if got.size else 0.0
    tol = PARITY_TOL[c.kv_dtype]
    return {"max_abs_err": err, "tol": tol, "values": int(got.size), "finite": finite,
            "pass": finite and err <= tol, "oracle_seconds": round(dt, 2),
            "compared": "every (sequence, query head, dim) output of the last timed step"}


def cpu_baseline(wl: Workload, budget_s: float) -> dict:
    """The fp64 oracle on a bounded sample of (sequence, head) pairs of the same
    workload, extrapolated to the whole batch by cached-token count."""
    from oracle import oracle as O

    c = wl.case
    threads = max(1, min(16, os.cpu_count() or 1))
    rng = np.random.default_rng(0)
    order = rng.permutation(c.B * c.Hq)
    pairs_all = np.stack([order // c.Hq, order % c.Hq], axis=1).astype(np.int32)
    n, used, t_used = threads, 0, 0.0
    while True:
        pairs = pairs_all[:n]
        t0 = time.perf_counter()
        O.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seqlens, c.scale,
                            kv_dtype=c.kv_dtype, block_size=c.bs, num_kv_heads=c.Hkv,
                            layout=c.layout, pairs=pairs, nthreads=threads)
        dt = time.perf_counter() - t0
        used, t_used = n, dt
        if dt > budget_s / 3 or n >= len(pairs_all):
            break
        n = min(len(pairs_all), int(n * max(2.0, budget_s / 3 / max(dt, 1e-3))))
    if used == len(pairs_all):  # the whole batch fits the budget: best of up to 3 runs
        for _ in range(2):
            if t_used * 2 > budget_s:
                break
            t0 = time.perf_counter()
            O.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seqlens, c.scale,
                                kv_dtype=c.kv_dtype, block_size=c.bs, num_kv_heads=c.Hkv,
                                layout=c.layout, pairs=pairs_all, nthreads=threads)
            t_used = min(t_used, time.perf_counter() - t0)
    tok_sample = int(c.seqlens[pairs_all[:used, 0]].astype(np.int64).sum())
    tok_all = int(c.seqlens.astype(np.int64).sum()) * c.Hq
    t_full = t_used * tok_all / tok_sample
    # one thread on a slice of the same sample, sized to about a sixth of the budget
    n1 = max(1, min(used, int(used * (budget_s / 6) / max(t_used * threads, 1e-3))))
    t0 = time.perf_counter()
    O.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seqlens, c.scale,
                        kv_dtype=c.kv_dtype, block_size=c.bs, num_kv_heads=c.Hkv,
                        layout=c.layout, pairs=pairs_all[:n1], nthreads=1)
    t1 = time.perf_counter() - t0
    tok1 = int(c.seqlens[pairs_all[:n1, 0]].astype(np.int64).sum())
    t1_full = t1 * tok_all / max(tok1, 1)
    return {"value": round(wl.kv_bytes / t_full / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": {"value": round(wl.kv_bytes / t1_full / 1e9, 4), "unit": "GB/s",
                              "sample": f"{n1} pairs ({tok1} head-tokens) in {t1:.2f}s"},
            "sample": f"{used} of {c.B * c.Hq} (sequence, query head) pairs of {c.name} "
                      f"({tok_sample} of {tok_all} head-tokens) in {t_used:.2f}s, "
                      "extrapolated by head-token count (best of up to 3 runs when the whole batch fits)",
            "seq_heads_per_s": round(c.B * c.Hq / t_full, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--also", type=str, default="3,5,1,2",
                    help="comma-separated extra configs ('' for none); 1 and 2 fit in the caches "
                         "and are reported for information")
    ap.add_argument("--path", default="auto", choices=["auto", "valu", "mfma", "mfma_grid", "mfma_stream",
                                                   "mfma_fused"])
    ap.add_argument("--partition", type=int, default=None,
                    help="partition size of every decode workload (default: the library's "
                         "choice, 512 for the 100K-token workload)")
    ap.add_argument("--layout", default="HND", choices=["HND", "XPACKED"],
                    help="K/V cache layout of the decode workloads (XPACKED: K [NB, H_kv, d/8, "
                         "bs, 8], V [NB, H_kv, d, bs], the same values)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the plain read-rate probes")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context legs (G sweep, one-shard shape, Qwen2 batch sweep)")
    ap.add_argument("--num-q-heads", type=int, default=None,
                    help="with --profile: keep the first N query heads of each sequence "
                         "(G = N / H_kv) of the workload")
    ap.add_argument("--profile", choices=["partition", "both", "copy", "prefill"], default=None)
    ap.add_argument("--prefill", type=str, default="1,2",
                    help="comma-separated prefill workloads to time ('' for none)")
    a = ap.parse_args()

    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (this "
              "decode path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if a.profile == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes x {a.steps}")
        return

    if a.profile == "prefill":  # the prefill workloads named by --prefill
        for k in [int(x) for x in a.prefill.split(",") if x.strip()]:
            measure_prefill(k, torch, a.steps, a.warmup)
        return

    case = None
    if a.num_q_heads is not None:
        from paged_gqa_decode_block_amd import workload as W

        case = W.make_config(a.config)
        hq = a.num_q_heads
        if hq % case.Hkv or hq > case.Hq:
            sys.exit(f"--num-q-heads must be a multiple of {case.Hkv} up to {case.Hq}")
        case = W.Case(**{**case.__dict__, "q": np.ascontiguousarray(case.q[:, :hq]), "Hq": hq,
                         "name": f"{case.name}_G{hq // case.Hkv}"})
    wl = Workload(a.config, torch, a.path, a.partition, a.layout, case=case)
    if a.profile is not None:
        for _ in range(a.warmup):
            wl.call()
        torch.cuda.synchronize()
        for _ in range(a.steps):
            wl.call(a.profile)
        torch.cuda.synchronize()
        log(f"[bench] {a.steps} '{a.profile}' launches of {wl.case.name} done")
        return

    flush_buf = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB > 256 MB MALL
    r = measure(wl, a.steps, a.warmup, flush_buf)
    got = wl.out.float().cpu().numpy()  # the last timed step's output
    r.update(measure_append_graph(wl, a.steps))
    log(f"[bench] {wl.case.name}: append + decode step as a graph replay "
        f"{r['append_graph_step_us']:.1f} us (output equals the plain step: {r['append_output_equals_decode']})")
    log(f"[bench] {wl.case.name}: {r['ms_per_step'] * 1e3:.1f} us/step flushed "
        f"({r['warm_ms_per_step'] * 1e3:.1f} warm), {r['kv_gbs']:.0f} GB/s")
    rl = roofline(wl, r)
    context = {}
    if not a.no_context:
        context["gqa_bytes_vs_G"] = gqa_sweep(wl, max(10, a.steps // 2), a.warmup, flush_buf)
    also = {}
    for k in [int(x) for x in a.also.split(",") if x.strip()]:
        if k == a.config:
            continue
        w2 = Workload(k, torch, a.path, a.partition, a.layout)
        r2 = measure(w2, a.steps, a.warmup, flush_buf)
        log(f"[bench] {w2.case.name}: {r2['ms_per_step'] * 1e3:.1f} us/step flushed "
            f"({r2['warm_ms_per_step'] * 1e3:.1f} warm), {r2['kv_gbs']:.0f} GB/s")
        also[w2.case.name] = {**w2.describe(), **{k2: (round(v, 4) if isinstance(v, float) else v)
                                                  for k2, v in r2.items()},
                              # on distinct K/V bytes (a shared block once): the
                              # logical rate of a prefix-shared batch read with
                              # folding can pass the HBM peak
                              "pct_hbm_peak": round(100 * r2["unique_kv_gbs"] / HBM_PEAK_GBS, 2),
                              "roofline": roofline(w2, r2)}
        if not a.no_cpu_baseline:
            also[w2.case.name]["parity"] = cpu_baseline_parity(w2, w2.out.float().cpu().numpy())
            log(f"[bench] {w2.case.name}: max-abs error vs the oracle "
                f"{also[w2.case.name]['parity']['max_abs_err']:.2e}")
        del w2
        torch.cuda.empty_cache()
    if not a.no_context:
        context["one_shard_of_8"] = shard_leg(torch, a.steps, a.warmup, flush_buf)
        context["qwen2_batch_sweep"] = batch_sweep(torch, a.steps, a.warmup, flush_buf)
    prefill = {}
    for k in [int(x) for x in a.prefill.split(",") if x.strip()]:
        r3 = measure_prefill(k, torch, max(5, a.steps // 5), 3)
        prefill[r3["workload"]] = r3
    probe = None
    if not a.no_probe:
        probe = read_probe(torch)
        probe["decode_kernel_vs_stream_read"] = round(rl["achieved"] / probe["stream_read_gbs"], 4)
        # against the gather of the workload's own K tile size (one block of one KV head)
        tile_kb = wl.case.bs * wl.case.D * (4 if wl.case.kv_dtype == "f32" else 2) // 1024
        if tile_kb in (4, 8):
            probe["decode_kernel_vs_tile_gather"] = round(
                rl["achieved"] / probe[f"tile_gather_{tile_kb}k_gbs"], 4)
        log(f"[bench] plain reads: {probe['stream_read_gbs']:.0f} GB/s sequential, "
            f"{probe['tile_gather_4k_gbs']:.0f} / {probe['tile_gather_8k_gbs']:.0f} GB/s as 4 / 8 KB tiles")
    cpu = None
    parity = None
    if not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(wl, a.cpu_seconds)
        parity = cpu_baseline_parity(wl, got)
        log(f"[bench] {wl.case.name}: max-abs error vs the oracle {parity['max_abs_err']:.2e}")
    line = {
        "metric": METRIC,
        "value": round(r["kv_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.case.kv_dtype,
        "data": "synthetic (seeded)",
        "config": wl.describe(),
        "pct_hbm_peak": round(100 * r["unique_kv_gbs"] / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(r["seq_heads_per_s"], 1),
        "detail": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()},
        "roofline": rl,
        "cpu_baseline": cpu,
        "max_abs_err": None if parity is None else parity["max_abs_err"],
        "parity": parity,
        "read_probe": probe,
        "also": also,
        "context": context,
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
