"""Benchmark of the single-token decode-attention hot path on one MI355X.

A step is one pass of the whole hot path over the long-context workload
(batch 8, 32 query heads sharing 8 KV heads, head_dim 128, bf16, kv_len 32768
= the full capacity, 1 % of key rows scaled x8): one ada_decode_step call that
appends the new key and value rows at the last slot (the append is folded
into the partial kernel), picks the split plan on the host, streams all
32768 slots of every (batch row, KV head) in the split-KV partial kernel and
merges the splits in the combine kernel. A call reads 1.07 GB, four times
the 256 MB Infinity Cache, so every step streams from HBM. The grouped-query
decode this workload stresses is the one the pages measure at a K width of
32768 (fish-speech PR #1337, "Isolated SDPA-kernel benchmark").

Printed: one JSON line with the metric (achieved algorithmic GB/s of the
timed steps), the roofline of the dominant kernel (the partial kernel:
algorithmic bytes / its average duration over back-to-back launches bracketed
by HIP events on the launching stream, with the host queued ahead so that
launch cost does not count, against 8 TB/s; traffic from the committed
rocprofv3 counter summary), the fp64 CPU oracle timed on the host cores,
and, under "also": every graded point against its 70 %-of-peak bar (the MHA
sweep at kv_len 4096 and 8192, the MiniCPM shape at positions 4095 and 8191
and its ragged draws, this workload), a streaming-read floor at the same
sizes, the 36-layer S2-Pro-shaped run, the MiniCPM lockstep sweep, the
full-capacity against active-prefix comparison, the decode step with rotary
embedding, one GPU's share under an 8-way split, and the causal prompt
prefill.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--long-context-only] [--only SECTIONS] [--prefill-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as W  # noqa: E402

METRIC = "q_len=1 GQA decode attention: µs/call and achieved HBM GB/s (% of peak)"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
MALL_BYTES = 256 * 2**20
CALIB_BYTES = 256 * 2**20  # calibration copy for the counter runs
SPIN_CYCLES = 100_000_000  # GPU-side spin (about 40 ms) that lets the host run ahead
SWEEP = (1024, 4096, 8192)
KERNEL_SOURCE = ROOT / "autoregressive_decode_attention_amd" / "csrc" / "ada_kernels.hip"
PMC_SUMMARY = ROOT / "profiles" / "decode_kernel_long_context_pmc.md"
ROOFLINE_MIN_LAUNCHES = 100
# Sections of "also" (bench.py --only picks some).
SECTIONS = ("mha_sweep", "minicpm_stream", "read_floor", "graded", "shards", "s2pro_run",
            "full_capacity_vs_active_prefix", "minicpm_sweep", "rope_step", "prefill")


# ---------------------------------------------------------------------------
# Byte model (algorithmic bytes: every live K and V element once per KV head,
# q read once, output written once; the split workspace is overhead, not
# algorithmic).


def kv_bytes(n_kv_head: int, head_dim: int, total_len: int, elem: int = 2) -> int:
    """K and V bytes of ``total_len`` live slots summed over batch rows."""
    return 2 * n_kv_head * head_dim * elem * total_len


def decode_bytes(batch: int, n_head: int, n_kv_head: int, head_dim: int, lens, elem: int = 2) -> int:
    return kv_bytes(n_kv_head, head_dim, sum(lens), elem) + 2 * batch * n_head * head_dim * elem


def append_bytes(batch: int, n_kv_head: int, head_dim: int, elem: int = 2) -> int:
    """New K and V rows read once and written once."""
    return 4 * batch * n_kv_head * head_dim * elem


def kernel_source_hash() -> str:
    return hashlib.sha256(KERNEL_SOURCE.read_bytes()).hexdigest()[:16]


def pmc_traffic() -> float | None:
    """HBM bytes (reads + writes) of one partial-kernel launch of the
    long-context workload from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since the counters
    were taken."""
    if not PMC_SUMMARY.exists():
        return None
    text = PMC_SUMMARY.read_text()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def bar_us(nbytes: int, frac: float = 0.7) -> float:
    """Duration at ``frac`` of the 8 TB/s peak for ``nbytes`` bytes."""
    return nbytes / (frac * PEAK_HBM_GBS * 1e3)


def device_timed(fn, iters: int) -> float:
    """Average device time (us) of ``iters`` back-to-back calls of fn(i),
    bracketed by HIP events on the current stream; a GPU-side spin queued
    first lets the host enqueue every call before the first runs, so host
    launch cost does not show up as gaps."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    a.record()
    for i in range(iters):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / iters


class LongContext:
    """The long-context workload: batch 8, 32/8 heads, head_dim 128, bf16,
    kv_len 32768 = capacity, 1 % of key rows x8 (the outlier rows stress the
    softmax range). One step = ada_decode_step appending at the last slot and
    attending over all 32768 slots (append folded into the partial kernel,
    host split plan, partial kernel, combine kernel)."""

    def __init__(self, ada, device):
        self.ada = ada
        wl = W.WORKLOADS["long_context"]
        self.shape = shp = wl.shape
        B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
        x = W.decode_inputs(shp, [S] * B, W.seed_for(4), device=device, tail="random",
                            outlier_p=wl.outlier_p, outlier_scale=wl.outlier_scale)
        self.q, self.k_cache, self.v_cache = x["q"], x["k_cache"], x["v_cache"]
        self.k_new, self.v_new = W.append_inputs(B, Hkv, D, shp.dtype, W.seed_for(4, 1), device=device)
        self.pos = S - 1
        self.splits, self.chunk = ada.decode_plan(B, Hq, Hkv, S)
        self.ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, self.splits)), device)
        self.out = torch.empty_like(self.q)
        self.scale = 1.0 / math.sqrt(D)
        self.partial_bytes = kv_bytes(Hkv, D, B * S) + B * Hq * D * 2  # K, V and q read
        self.call_bytes = decode_bytes(B, Hq, Hkv, D, [S] * B)
        self.step_bytes = self.call_bytes + append_bytes(B, Hkv, D)

    def step(self, i: int = 0):
        self.ada.decode_step(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache, self.pos,
                             scale=self.scale, out=self.out, workspace=self.ws)

    def partial(self, i: int = 0):
        self.ada.decode_partial(self.q, self.k_cache, self.v_cache, None, scale=self.scale,
                                max_kv_len=self.shape.capacity, workspace=self.ws)


# ---------------------------------------------------------------------------


class Sweep:
    """The one-token MHA decode sweep of Cuda-Compute-OSS #343 ("Current
    limitation"): batch 1, 16 query heads = 16 KV heads, head_dim 128, fp16,
    kv_len 1024 / 4096 / 8192, each with its own caches, rotated over enough
    sets (960 MiB) that no call finds its K/V in the 256 MB Infinity Cache."""

    def __init__(self, ada, device, sets: int | None = None):
        self.ada = ada
        wl = W.WORKLOADS["mha_sweep"]
        self.shape = shp = wl.shape
        B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
        per_call = [kv_bytes(Hkv, D, B * n) for n in SWEEP]
        per_step = sum(per_call)
        self.sets = sets or max(2, math.ceil(2 * MALL_BYTES / per_step))
        self.caches = []  # [set][kv index] -> (k, v)
        for s in range(self.sets):
            row = []
            for j, n in enumerate(SWEEP):
                x = W.decode_inputs(shp, [n], W.seed_for(1, 100 * s + j), device=device, tail="random")
                row.append((x["k_cache"], x["v_cache"]))
            self.caches.append(row)
        self.q = [W.randn16((B, Hq, D), shp.dtype, W.seed_for(1, 7000 + j), device=device) for j in range(3)]
        self.out = [torch.empty((B, Hq, D), dtype=W.TORCH_DTYPES[shp.dtype], device=device) for _ in SWEEP]
        self.scale = 1.0 / math.sqrt(D)
        self.decode_bytes = [decode_bytes(B, Hq, Hkv, D, [n]) for n in SWEEP]
        ws_need = max(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, ada.decode_num_splits(B, Hq, Hkv, n)))
                      for n in SWEEP)
        self.ws = ada.new_workspace(ws_need, device)

    def time_partials(self, iters: int) -> list:
        """Average duration of the partial kernel per kv_len: ``iters`` launches
        back to back (rotating cache sets), bracketed by HIP events on the
        launching stream. A GPU-side spin queued first lets the host enqueue
        every launch before the first one runs, so host launch cost does not
        show up as gaps."""
        ada = self.ada
        res = []
        for j, n in enumerate(SWEEP):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(SPIN_CYCLES)
            a.record()
            for i in range(iters):
                k, v = self.caches[i % self.sets][j]
                ada.decode_partial(self.q[j], k, v, None, scale=self.scale, max_kv_len=n, workspace=self.ws)
            b.record()
            torch.cuda.synchronize()
            res.append(a.elapsed_time(b) * 1e3 / iters)
        return res

    def time_calls(self, iters: int, resident: bool = False) -> list:
        """As time_partials, for whole decode calls (partial + combine). With
        ``resident`` every call reads the same cache set, which then stays in
        the 256 MB Infinity Cache: a cache-resident figure, not an HBM one."""
        ada = self.ada
        res = []
        for j, n in enumerate(SWEEP):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if resident:
                k, v = self.caches[0][j]
                for _ in range(3):
                    ada.decode_partial(self.q[j], k, v, None, scale=self.scale, max_kv_len=n, workspace=self.ws)
            torch.cuda.synchronize()
            torch.cuda._sleep(SPIN_CYCLES)
            a.record()
            for i in range(iters):
                k, v = self.caches[0 if resident else i % self.sets][j]
                _, used = ada.decode_partial(self.q[j], k, v, None, scale=self.scale, max_kv_len=n,
                                             workspace=self.ws)
                ada.decode_combine(self.ws, used, self.out[j], self.shape.n_kv_head)
            b.record()
            torch.cuda.synchronize()
            res.append(a.elapsed_time(b) * 1e3 / iters)
        return res


def time_shards(ada, device, iters: int = 20) -> dict:
    """One GPU's share of the long-context workload under two 8-way splits
    (the exchange between GPUs is not measured here): (a) KV heads over 8
    GPUs -- batch 8, 4 query heads sharing 1 KV head, kv_len 32768, one whole
    decode call; (b) the sequence over 8 GPUs -- each holds 4096 slots of
    every (batch row, KV head) and runs the partial kernel on them, then,
    once the partials are all-gathered, one combine over 8x its own split
    count (timed on partials of the same size)."""
    wl = W.WORKLOADS["long_context"]
    shp = wl.shape
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    scale = 1.0 / math.sqrt(D)

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    res = {}
    tp = W.DecodeShape(B, Hq // 8, Hkv // 8, D, S, shp.dtype)
    x = W.decode_inputs(tp, [S] * B, W.seed_for(4, 90_000), device=device, tail="random",
                        outlier_p=wl.outlier_p, outlier_scale=wl.outlier_scale)
    splits = ada.decode_num_splits(B, tp.n_head, tp.n_kv_head, S)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, tp.n_head, tp.n_kv_head, D, max(2, splits)), device)
    out = torch.empty_like(x["q"])
    us = timed(lambda: ada.decode_attn_gqa(x["q"], x["k_cache"], x["v_cache"], None, scale=scale, out=out,
                                           max_kv_len=S, workspace=ws))
    nb = decode_bytes(B, tp.n_head, tp.n_kv_head, D, [S] * B)
    res["kv_heads_over_8"] = {"shape": "batch 8, 4/1 heads, kv_len 32768, bf16", "splits": splits,
                              "call_us": round(us, 2), "GBs": round(nb / us / 1e3, 1),
                              "frac_of_peak": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    del x
    n = S // 8
    sp = W.DecodeShape(B, Hq, Hkv, D, n, shp.dtype)
    x = W.decode_inputs(sp, [n] * B, W.seed_for(4, 90_001), device=device, tail="random",
                        outlier_p=wl.outlier_p, outlier_scale=wl.outlier_scale)
    local = ada.decode_num_splits(B, Hq, Hkv, n)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, 8 * local), device)
    out = torch.empty_like(x["q"])
    part = timed(lambda: ada.decode_partial(x["q"], x["k_cache"], x["v_cache"], None, scale=scale, max_kv_len=n,
                                            workspace=ws))
    ada.decode_partial(x["q"], x["k_cache"], x["v_cache"], None, scale=scale, max_kv_len=n,
                       num_splits=8 * local, workspace=ws)
    comb = timed(lambda: ada.decode_combine(ws, 8 * local, out, Hkv))
    nb = decode_bytes(B, Hq, Hkv, D, [n] * B)
    res["sequence_over_8"] = {"shape": "batch 8, 32/8 heads, 4096 of 32768 slots per GPU, bf16",
                              "local_splits": local, "partial_us": round(part, 2),
                              "partial_GBs": round(nb / part / 1e3, 1),
                              "combine_us_over_8x_splits": round(comb, 2),
                              "partial_bytes_per_gpu_to_gather": B * Hq * local * (D + 2) * 4}
    del x
    return res


def time_s2pro_run(ada, device) -> dict:
    """The S2-Pro-shaped run (36 layers, 32/8 heads, fp16, capacity 32768,
    prefill 234, then 1024 decode steps): one HIP graph holds a whole decode
    step -- per layer one ada_decode_step (append at slot 234 + i and attend
    over 235 + i slots) -- plus the library's device-side increment of the
    position (ada_step_graph_create), so one launch per step runs the whole
    run with no host work in between.
    Timed over all 1024 replays (36 864 decode calls)."""
    wl = W.WORKLOADS["s2pro_run"]
    shp = wl.shape
    L, T0, N = wl.layers, wl.prefill, wl.steps
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    last = T0 + N
    dt = W.TORCH_DTYPES[shp.dtype]
    kc = torch.zeros((L, B, Hkv, S, D), dtype=dt, device=device)
    vc = torch.zeros_like(kc)
    for layer in range(L):
        x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, T0, shp.dtype), [T0], W.seed_for(2, layer),
                            device=device, tail="random")
        kc[layer, :, :, :T0] = x["k_cache"]
        vc[layer, :, :, :T0] = x["v_cache"]
    k_new = W.randn16((L, B, Hkv, D), shp.dtype, W.seed_for(2, 20_000), device=device)
    v_new = W.randn16((L, B, Hkv, D), shp.dtype, W.seed_for(2, 20_001), device=device)
    q = W.randn16((L, B, Hq, D), shp.dtype, W.seed_for(2, 20_002), device=device)
    out = torch.empty((L, B, Hq, D), dtype=dt, device=device)
    pos = torch.full((B,), T0, dtype=torch.int32, device=device)
    splits = ada.decode_num_splits(B, Hq, Hkv, last)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, splits)), device)
    scale = 1.0 / math.sqrt(D)

    # One library graph: every layer's ada_decode_step, then the position
    # advance, recorded once (ada_step_graph_create) and replayed per step.
    layers = [(q[layer], k_new[layer], v_new[layer], kc[layer], vc[layer], out[layer]) for layer in range(L)]
    graph = ada.step_graph(layers, pos, last - 1, scale=scale, workspace=ws)
    graph.launch()  # warm-up replay
    pos.fill_(T0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(N):
        graph.launch()
    torch.cuda.synchronize()
    run_ms = (time.perf_counter() - t0) * 1e3
    graph.close()
    nbytes = L * sum(decode_bytes(B, Hq, Hkv, D, [n]) for n in range(T0 + 1, last + 1))
    del kc, vc
    return {"workload": "s2pro_run: 36 layers, 32/8 heads, head_dim 128, fp16, capacity 32768, prefill 234, "
                        "1024 steps (kv_len 235..1258), one decode step (append + attend) per layer, one graph replay per step",
            "run_ms": round(run_ms, 2), "ms_per_step": round(run_ms / N, 4),
            "us_per_layer_call": round(run_ms * 1e3 / (N * L), 2), "run_bytes": nbytes,
            "GBs": round(nbytes / (run_ms * 1e-3) / 1e9, 1), "splits": splits}


def time_minicpm_sweep(ada, device, layers: int = 4) -> dict:
    """The MiniCPM-shaped lockstep sweep (batch 4, 32/8 heads, bf16, capacity
    8192; VoxCPM #395, section 6.3): position_id swept 0..8191, each step
    appending the new rows at slot p and attending over p + 1 slots. One
    library step graph holds ``layers`` layers (separate caches, together
    above the 256 MB Infinity Cache, so the reads come from HBM) and the
    device-side position advance; one replay per position, 8192 replays.
    The launches are sized for the last slot (max_pos 8191) and the positions
    live on the device, so the balanced plan spreads each step's rows over
    the splits."""
    shp = W.WORKLOADS["minicpm_stream"].shape
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    L = layers
    dt = W.TORCH_DTYPES[shp.dtype]
    kc = torch.empty((L, B, Hkv, S, D), dtype=dt, device=device)
    vc = torch.empty_like(kc)
    for layer in range(L):
        x = W.decode_inputs(shp, [S] * B, W.seed_for(3, 80_000 + layer), device=device, tail="random")
        kc[layer].copy_(x["k_cache"])
        vc[layer].copy_(x["v_cache"])
        del x
    k_new = W.randn16((L, B, Hkv, D), shp.dtype, W.seed_for(3, 81_000), device=device)
    v_new = W.randn16((L, B, Hkv, D), shp.dtype, W.seed_for(3, 81_001), device=device)
    q = W.randn16((L, B, Hq, D), shp.dtype, W.seed_for(3, 81_002), device=device)
    out = torch.empty((L, B, Hq, D), dtype=dt, device=device)
    pos = torch.zeros((B,), dtype=torch.int32, device=device)
    splits = ada.decode_num_splits(B, Hq, Hkv, S)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, splits)), device)
    graph = ada.step_graph([(q[i], k_new[i], v_new[i], kc[i], vc[i], out[i]) for i in range(L)], pos, S - 1,
                           scale=1.0 / math.sqrt(D), workspace=ws)
    graph.launch()  # warm-up replay
    pos.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(S):
        graph.launch()
    torch.cuda.synchronize()
    run_ms = (time.perf_counter() - t0) * 1e3
    graph.close()
    nbytes = L * sum(decode_bytes(B, Hq, Hkv, D, [p + 1] * B) for p in range(S))
    del kc, vc
    return {"workload": f"minicpm lockstep sweep: batch 4, 32/8 heads, head_dim 128, bf16, capacity 8192, positions "
                        f"0..8191, {L} layers (one decode step each) per graph replay",
            "run_ms": round(run_ms, 2), "us_per_layer_call": round(run_ms * 1e3 / (S * L), 2), "run_bytes": nbytes,
            "GBs": round(nbytes / (run_ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (run_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "splits": splits}


def time_full_vs_active(ada, device, iters: int = 20) -> dict:
    """The pages' experiment restated on this kernel (fish-speech #1310,
    "CUDA benchmark"; VoxCPM #395, section 6.3): a decode call that attends
    over the whole preallocated capacity (what a full-width mask costs: every
    slot is read) against one over the live prefix only, at the S2-Pro shape
    (capacity 32768, live 235 and 1258) and the MiniCPM shape (batch 4,
    capacity 8192, live 1522 and 5617, two of that page's sampled positions).
    Caches rotate so every call reads HBM."""
    cases = [("s2pro", W.WORKLOADS["s2pro_run"].shape, (235, 1258)),
             ("minicpm", W.WORKLOADS["minicpm_stream"].shape, (1522, 5617))]
    res = {}
    for name, shp, lives in cases:
        B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
        per_full = kv_bytes(Hkv, D, B * S)
        R = max(2, math.ceil(2 * MALL_BYTES / per_full))
        xs = [W.decode_inputs(shp, [S] * B, W.seed_for(2, 30_000 + r), device=device, tail="random") for r in range(R)]
        ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, 256), device)
        out = torch.empty_like(xs[0]["q"])

        def timed(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(SPIN_CYCLES)
            a.record()
            for i in range(iters):
                x = xs[i % R]
                ada.decode_attn_gqa(x["q"], x["k_cache"], x["v_cache"], None, max_kv_len=n, out=out, workspace=ws)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / iters

        full = timed(S)
        row = {"capacity": S, "full_capacity_us": round(full, 2)}
        for n in lives:
            us = timed(n)
            row[f"live_{n}_us"] = round(us, 2)
            row[f"speedup_at_{n}"] = round(full / us, 2)
        res[name] = row
        del xs
    return res


def time_rope_step(ada, device, iters: int = 100) -> dict:
    """The decode step with rotary embedding (VoxCPM #395, section 4: rotate
    the step's query and key, write the cache rows at position_id, attend over
    0..position_id) at the MiniCPM shape (batch 4, 32/8 heads, bf16, capacity
    8192, lockstep positions 4095 and 8191): ada_decode_step_rope against the
    plain ada_decode_step, and the standalone ada_rope_kv_append, each averaged
    over back-to-back calls bracketed by HIP events, caches rotated so every
    call reads HBM."""
    shp = W.WORKLOADS["minicpm_stream"].shape
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    R = max(2, math.ceil(2 * MALL_BYTES / kv_bytes(Hkv, D, B * S)))
    xs = [W.decode_inputs(shp, [S] * B, W.seed_for(3, 40_000 + r), device=device, tail="random") for r in range(R)]
    k_new, v_new = W.append_inputs(B, Hkv, D, shp.dtype, W.seed_for(3, 41_000), device=device)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, 256), device)
    out = torch.empty_like(xs[0]["q"])
    q_rot = torch.empty_like(xs[0]["q"])
    scale = 1.0 / math.sqrt(D)

    def timed(fn):
        fn(0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        a.record()
        for i in range(iters):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    res = {"workload": "minicpm shape: batch 4, 32/8 heads, head_dim 128, bf16, capacity 8192, lockstep position p",
           "launches": "decode_step and decode_step_rope: 2 each; rope_kv_append: 1"}
    for p in (4095, 8191):
        cos, sin = W.rope_tables([p] * B, D, shp.dtype, device=device)
        pos_t = torch.full((B,), p, dtype=torch.int32, device=device)

        def plain(i, p=p):
            x = xs[i % R]
            ada.decode_step(x["q"], k_new, v_new, x["k_cache"], x["v_cache"], p, scale=scale, out=out, workspace=ws)

        def rope(i, p=p, cos=cos, sin=sin):
            x = xs[i % R]
            ada.decode_step_rope(x["q"], k_new, v_new, cos, sin, x["k_cache"], x["v_cache"], p, scale=scale,
                                 out=out, workspace=ws)

        def append_only(i, cos=cos, sin=sin, pos_t=pos_t):
            x = xs[i % R]
            ada.rope_kv_append(x["q"], k_new, v_new, cos, sin, x["k_cache"], x["v_cache"], pos_t, q_out=q_rot)

        nbytes = decode_bytes(B, Hq, Hkv, D, [p + 1] * B)
        t_plain, t_rope, t_app = timed(plain), timed(rope), timed(append_only)
        res[f"p{p}"] = {"bytes_per_call": nbytes, "decode_step_us": round(t_plain, 2),
                        "decode_step_rope_us": round(t_rope, 2), "rope_overhead_us": round(t_rope - t_plain, 2),
                        "decode_step_rope_GBs": round(nbytes / t_rope / 1e3, 1),
                        "rope_kv_append_us": round(t_app, 2)}
    del xs
    return res


def time_minicpm_stream(ada, device, iters: int = 50, draws: int = 64) -> dict:
    """The MiniCPM-shaped streaming workload (batch 4, 32/8 heads, bf16,
    capacity 8192; VoxCPM #395, sections 2.2 and 6.3): (a) lockstep decode
    steps (append at position p, attend over p + 1 slots) at p = 4095 and
    8191, with one host position for the batch and again with the positions
    in a device tensor and the launch sized for the last slot (max_pos 8191,
    as a captured decode loop has it: the balanced plan); (b) ragged batches,
    per-row kv_len drawn uniformly from [1, 8192] (seeded), lengths on the
    device. Each figure is the average over back-to-back calls bracketed by
    HIP events, with caches rotated so every call reads HBM; GB/s counts the
    live slots only."""
    shp = W.WORKLOADS["minicpm_stream"].shape
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    R = max(2, math.ceil(2 * MALL_BYTES / kv_bytes(Hkv, D, B * S)))
    xs = [W.decode_inputs(shp, [S] * B, W.seed_for(3, 70_000 + r), device=device, tail="random") for r in range(R)]
    k_new, v_new = W.append_inputs(B, Hkv, D, shp.dtype, W.seed_for(3, 71_000), device=device)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, 256), device)
    out = torch.empty_like(xs[0]["q"])
    scale = 1.0 / math.sqrt(D)

    def timed(fn):
        fn(0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        a.record()
        for i in range(iters):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    res = {"workload": "minicpm_stream: batch 4, 32/8 heads, head_dim 128, bf16, capacity 8192"}
    for p in (4095, 8191):
        us = timed(lambda i, p=p: ada.decode_step(xs[i % R]["q"], k_new, v_new, xs[i % R]["k_cache"],
                                                  xs[i % R]["v_cache"], p, scale=scale, out=out, workspace=ws))
        nb = decode_bytes(B, Hq, Hkv, D, [p + 1] * B)
        res[f"lockstep_p{p}"] = {"bytes": nb, "us": round(us, 2), "GBs": round(nb / us / 1e3, 1),
                                 "frac_of_peak": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
        pt = torch.full((B,), p, dtype=torch.int32, device=device)
        us = timed(lambda i, pt=pt: ada.decode_step(xs[i % R]["q"], k_new, v_new, xs[i % R]["k_cache"],
                                                    xs[i % R]["v_cache"], pt, scale=scale, out=out, max_pos=S - 1,
                                                    workspace=ws))
        res[f"lockstep_p{p}_device_positions"] = {"us": round(us, 2), "GBs": round(nb / us / 1e3, 1),
                                                  "frac_of_peak": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    rows = []
    for d in range(draws):
        lens = W.ragged_lengths(B, 1, S, W.seed_for(3, 72_000 + d))
        lt = torch.tensor(lens, dtype=torch.int32, device=device)
        us = timed(lambda i, lt=lt: ada.decode_attn_gqa(xs[i % R]["q"], xs[i % R]["k_cache"], xs[i % R]["v_cache"],
                                                         lt, scale=scale, out=out, max_kv_len=S, workspace=ws))
        rows.append((lens, us, decode_bytes(B, Hq, Hkv, D, lens)))
    tot_b = sum(r[2] for r in rows)
    tot_us = sum(r[1] for r in rows)
    big = [r for r in rows if sum(r[0]) / B >= 4096]
    big_b, big_us = sum(r[2] for r in big), sum(r[1] for r in big)
    res["ragged"] = {"draws": draws, "mean_us": round(tot_us / draws, 2), "GBs": round(tot_b / tot_us / 1e3, 1),
                     "frac_of_peak": round(tot_b / tot_us / 1e3 / PEAK_HBM_GBS, 4),
                     "draws_mean_len_ge_4096": len(big),
                     "bytes_mean_len_ge_4096": big_b // max(1, len(big)),
                     "us_mean_len_ge_4096": round(big_us / max(1, len(big)), 2),
                     "GBs_mean_len_ge_4096": round(big_b / max(1e-9, big_us) / 1e3, 1)}
    del xs
    return res


PEAK_MFMA_16BIT_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak


def time_prefill(ada, device, iters: int = 30) -> dict:
    """Prompt prefill (fish-speech #1310, section 2: kv_len = T after the
    prompt; VoxCPM #395, section 5: causal attention): ada_prefill_attn_gqa
    from slot 0 over a prompt already in the cache, averaged over back-to-back
    launches bracketed by HIP events. Flops = 4 * D * H_q * B * T (T + 1) / 2
    (q.k and p.v over the visible slots only), against the dense 16-bit MFMA
    peak. Cases: the S2-Pro prompt (234 tokens, 32/8 heads, fp16, capacity
    32768) and a 4096-token prompt (32/8 heads, bf16, capacity 8192)."""
    res = {}
    for name, B, Hq, Hkv, T, S, dtype in (("s2pro_prompt", 1, 32, 8, 234, 32768, "fp16"),
                                          ("prompt_4096", 1, 32, 8, 4096, 8192, "bf16")):
        D = 128
        q = W.randn16((B, Hq, T, D), dtype, W.seed_for(2, 60_000), device=device)
        k = W.randn16((B, Hkv, S, D), dtype, W.seed_for(2, 60_001), device=device)
        v = W.randn16((B, Hkv, S, D), dtype, W.seed_for(2, 60_002), device=device)
        out = torch.empty_like(q)
        ada.prefill_attn_gqa(q, k, v, None, out=out)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        a.record()
        for _ in range(iters):
            ada.prefill_attn_gqa(q, k, v, None, out=out)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / iters
        flops = 4 * D * Hq * B * T * (T + 1) / 2
        tfs = flops / us / 1e6
        res[name] = {"workload": f"batch {B}, {Hq}/{Hkv} heads, head_dim {D}, {dtype}, prompt {T} tokens from slot 0, "
                                 f"capacity {S}",
                     "us": round(us, 2), "flops": int(flops), "TFLOPs": round(tfs, 1),
                     "frac_of_mfma_peak": round(tfs / PEAK_MFMA_16BIT_TFLOPS, 4)}
        del q, k, v, out
    return res


READ_FLOOR_POOL = 2 * 2**30  # bytes of the buffer the read probe rotates over


def time_read_floor(ada, device, sizes, iters: int = 20) -> list:
    """The streaming-read floor at each size (bytes): ada_hbm_read, the
    decode kernel's loads with no arithmetic, over a 2 GiB pool (calls rotate
    over disjoint regions, so sizes below the 256 MB Infinity Cache still
    come from HBM), at several workgroup counts; the best is reported."""
    pool = torch.empty(READ_FLOOR_POOL, dtype=torch.uint8, device=device)
    pool.fill_(1)
    sink = torch.empty(4 * 8192, dtype=torch.int32, device=device)
    rows = []
    for nbytes in sizes:
        nbytes = (int(nbytes) + 15) // 16 * 16
        regions = max(1, READ_FLOOR_POOL // nbytes)
        views = [pool[r * nbytes:(r + 1) * nbytes] for r in range(min(regions, 64))]
        best = None
        for wgs in (256, 512, 1024, 2048, 4096, 8192):
            ada.hbm_read(views[0], sink, wgs)
            us = device_timed(lambda i, wgs=wgs: ada.hbm_read(views[i % len(views)], sink, wgs), iters)
            if best is None or us < best[1]:
                best = (wgs, us)
        rows.append({"bytes": nbytes, "best_workgroups": best[0], "us": round(best[1], 2),
                     "GBs": round(nbytes / best[1] / 1e3, 1),
                     "frac_of_peak": round(nbytes / best[1] / 1e3 / PEAK_HBM_GBS, 4),
                     "regions_rotated": len(views)})
    del pool, sink
    return rows


def graded_points(lc_call_us: float, lc_bytes: int, per_kv: list, minicpm: dict, floor: list) -> list:
    """Every point the 70 %-of-peak target applies to (kv_len >= 4096): bytes
    per call, the bar (duration at 70 % of 8 TB/s), the measured whole-call
    duration and its fraction of peak, and the streaming-read floor of the
    same bytes."""
    fl = {r["bytes"]: r for r in floor}

    def row(name, nbytes, us):
        f = fl.get((nbytes + 15) // 16 * 16)
        return {"point": name, "bytes": nbytes, "bar_us": round(bar_us(nbytes), 2), "us": round(us, 2),
                "frac_of_peak": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4), "meets_bar": us <= bar_us(nbytes),
                "read_floor_us": f["us"] if f else None}

    out = []
    for r in per_kv:
        if r["kv_len"] >= 4096:
            out.append(row(f"mha_sweep kv_len {r['kv_len']} (decode call)", r["bytes"], r["call_us"]))
    for p in (4095, 8191):
        m = minicpm[f"lockstep_p{p}"]
        out.append(row(f"minicpm_stream lockstep position {p} (decode step)", m["bytes"], m["us"]))
    rg = minicpm["ragged"]
    if rg["draws_mean_len_ge_4096"]:
        out.append(row(f"minicpm_stream ragged, {rg['draws_mean_len_ge_4096']} draws with mean kv_len >= 4096 "
                       "(decode call, mean)", rg["bytes_mean_len_ge_4096"], rg["us_mean_len_ge_4096"]))
    out.append(row("long_context (decode step)", lc_bytes, lc_call_us))
    return out


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline() -> dict:
    """The fp64 oracle (oracle/ada_oracle.c, OpenMP over (batch row, query
    head)) on the host cores, on the same seeded inputs as the GPU: the
    headline figure is one whole long-context call at nproc threads; beside
    it, every workload at 1 thread and at nproc threads (the long-context
    call at 1 thread on one of its 8 batch rows). GB/s counts the same
    algorithmic bytes as the GPU figures."""
    import oracle

    ora = oracle.load()
    nproc = os.cpu_count() or 1
    scale = 1.0 / math.sqrt(128)

    def case(name, shp, lens, seed, outliers=None):
        x = W.decode_inputs(W.DecodeShape(len(lens), shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity,
                                          shp.dtype), lens, seed, tail="random",
                            **({} if outliers is None else {"outlier_p": outliers[0], "outlier_scale": outliers[1]}))
        return name, x, lens, decode_bytes(len(lens), shp.n_head, shp.n_kv_head, shp.head_dim, lens)

    def run(x, lens, threads):
        ora.set_threads(threads)
        t = time.perf_counter()
        ora.decode(x["q"], x["k_cache"], x["v_cache"], lens, scale)
        return time.perf_counter() - t

    wl = W.WORKLOADS
    lc = wl["long_context"]
    cases = [case("tiny (kv_len 400)", wl["tiny"].shape, [400], W.seed_for(0))]
    for n in SWEEP:
        s2 = wl["mha_sweep"].shape
        cases.append(case(f"mha_sweep kv_len {n}", W.DecodeShape(1, s2.n_head, s2.n_kv_head, 128, n, s2.dtype), [n],
                          W.seed_for(1, n)))
    for n in (235, 1258):
        cases.append(case(f"s2pro_run one layer-call, kv_len {n}", wl["s2pro_run"].shape, [n], W.seed_for(2, n)))
    mc = wl["minicpm_stream"].shape
    cases.append(case("minicpm_stream lockstep position 8191", mc, [8192] * 4, W.seed_for(3, 8191)))
    cases.append(case("minicpm_stream ragged draw", mc, W.ragged_lengths(4, 1, mc.capacity, W.seed_for(3, 72_000)),
                      W.seed_for(3, 72_000)))
    lc_shape = lc.shape
    one_row = case("long_context, batch row 0 of 8", W.DecodeShape(1, lc_shape.n_head, lc_shape.n_kv_head, 128,
                                                                    lc_shape.capacity, lc_shape.dtype),
                   [lc_shape.capacity], W.seed_for(4), (lc.outlier_p, lc.outlier_scale))
    table = []
    for name, x, lens, nb in cases + [one_row]:
        t1 = run(x, lens, 1)
        tn = run(x, lens, nproc)
        table.append({"workload": name, "bytes": nb, "ms_1_thread": round(t1 * 1e3, 2),
                      "GBs_1_thread": round(nb / t1 / 1e9, 4), f"ms_{nproc}_threads": round(tn * 1e3, 2),
                      f"GBs_{nproc}_threads": round(nb / tn / 1e9, 4)})
    del cases, one_row
    name, x, lens, nb = case("long_context", lc_shape, [lc_shape.capacity] * lc_shape.batch, W.seed_for(4),
                             (lc.outlier_p, lc.outlier_scale))
    t = run(x, lens, nproc)
    ora.set_threads(nproc)
    return {"value": round(nb / t / 1e9, 4), "unit": "GB/s", "cores": nproc, "kind": "oracle",
            "sample": f"one whole long-context decode call (batch 8, 32/8 heads, kv_len 32768, bf16, "
                      f"{nb} algorithmic bytes) in {t:.2f} s at {nproc} threads; the cache append not included",
            "ms_per_call": round(t * 1e3, 1), "cpu_model": cpu_model(), "nproc": nproc,
            "per_workload": table}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--long-context-only", action="store_true",
                    help="the contract line of the long-context workload only (no other workloads, no step-graph "
                         "replays): for counter passes")
    ap.add_argument("--only", default=None,
                    help="comma-separated sections of 'also' to run (default: all): " + ", ".join(SECTIONS) +
                         "; graded and read_floor need mha_sweep and minicpm_stream")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prompt prefill cases and print them (for profiling runs); "
                         "no contract line")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode kernel needs no exchange between GPUs "
              "(batch rows and KV heads are independent); run with --gpus 1.", file=sys.stderr)
        return 2

    import autoregressive_decode_attention_amd as ada

    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    if args.prefill_only:
        print(json.dumps({"prefill": time_prefill(ada, device)}), flush=True)
        return 0
    # A plain copy of known size (256 MiB read, 256 MiB written): the reference
    # that scales the FETCH_SIZE / WRITE_SIZE counters of the profiled runs.
    calib_src = torch.empty(CALIB_BYTES // 2, dtype=torch.float16, device=device).fill_(1.0)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    lc = LongContext(ada, device)
    for _ in range(args.warmup):
        lc.step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        lc.step()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = lc.step_bytes / (ms_per_step * 1e-3) / 1e9
    step_dev_us = ev0.elapsed_time(ev1) * 1e3 / args.steps

    # Roofline of the dominant kernel: the partial kernel of the same call,
    # launched back to back; and the whole step the same way.
    n_roof = max(args.steps, ROOFLINE_MIN_LAUNCHES)
    lc.partial()
    part_us = device_timed(lc.partial, n_roof)
    call_us = device_timed(lc.step, n_roof)
    achieved = lc.partial_bytes / part_us / 1e3
    traffic = pmc_traffic()
    headline = {"step_us_events_timed_region": round(step_dev_us, 2),
                "step_us_back_to_back": round(call_us, 2), "step_launches_back_to_back": n_roof,
                "step_GBs_back_to_back": round(lc.step_bytes / call_us / 1e3, 1),
                "step_frac_of_peak_back_to_back": round(lc.step_bytes / call_us / 1e3 / PEAK_HBM_GBS, 4),
                "bar_us_70pct": round(bar_us(lc.step_bytes), 2), "splits": lc.splits, "chunk": lc.chunk}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "long_context: one-token GQA decode step, batch 8, 32 query heads / 8 KV heads, "
                               "head_dim 128, bf16, kv_len 32768 = capacity, 1% of key rows x8 (append at slot "
                               "32767, attend over 32768 slots)",
                   "step_bytes": lc.step_bytes, "kernels_per_step": 1 if lc.splits == 1 else 2,
                   "launch": "eager (ada_decode_step per step)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "traffic_basis": "HBM bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of one partial launch of "
                                      f"this workload; algorithmic bytes of that launch: {lc.partial_bytes}",
                     "kernel": "partial_kernel<bf16, G=4> (split-KV partial; the combine kernel follows it)",
                     "bytes_per_launch": lc.partial_bytes, "us_per_launch": round(part_us, 2),
                     "launches_timed": n_roof},
        "also": {"headline": headline},
    }
    wanted = set(SECTIONS) if args.only is None else {x for x in args.only.split(",") if x}
    unknown = wanted - set(SECTIONS)
    if unknown:
        print(f"unknown sections: {sorted(unknown)}", file=sys.stderr)
        return 2
    if args.long_context_only:
        wanted = set()
    also = line["also"]
    if "mha_sweep" in wanted:
        sweep = Sweep(ada, device)
        part_mha = sweep.time_partials(max(args.steps, ROOFLINE_MIN_LAUNCHES))
        call_mha = sweep.time_calls(max(args.steps, ROOFLINE_MIN_LAUNCHES))
        hot_mha = sweep.time_calls(max(args.steps, ROOFLINE_MIN_LAUNCHES), resident=True)
        per_kv = []
        for j, n in enumerate(SWEEP):
            nb = sweep.decode_bytes[j]
            per_kv.append({"kv_len": n, "bytes": nb, "splits": ada.decode_num_splits(1, 16, 16, n),
                           "partial_us": round(part_mha[j], 2), "partial_GBs": round(nb / part_mha[j] / 1e3, 1),
                           "call_us": round(call_mha[j], 2), "call_GBs": round(nb / call_mha[j] / 1e3, 1),
                           "call_frac_of_peak": round(nb / call_mha[j] / 1e3 / PEAK_HBM_GBS, 4),
                           "cache_resident_call_us": round(hot_mha[j], 2),
                           "cache_resident_call_GBs": round(nb / hot_mha[j] / 1e3, 1)})
        del sweep
        also["mha_sweep"] = per_kv
    if "minicpm_stream" in wanted:
        also["minicpm_stream"] = time_minicpm_stream(ada, device)
    lc_sizes = (lc.partial_bytes, lc.step_bytes)
    del lc
    if {"read_floor", "graded"} & wanted and {"mha_sweep", "minicpm_stream"} <= wanted:
        mc = also["minicpm_stream"]
        sizes = sorted({r["bytes"] for r in also["mha_sweep"] if r["kv_len"] >= 4096} |
                       {mc[f"lockstep_p{p}"]["bytes"] for p in (4095, 8191)} |
                       {mc["ragged"]["bytes_mean_len_ge_4096"], *lc_sizes})
        also["read_floor"] = time_read_floor(ada, device, sizes)
        also["graded"] = graded_points(call_us, line["config"]["step_bytes"], also["mha_sweep"], mc,
                                       also["read_floor"])
    for name, fn in (("shards", time_shards), ("s2pro_run", time_s2pro_run),
                     ("full_capacity_vs_active_prefix", time_full_vs_active), ("minicpm_sweep", time_minicpm_sweep),
                     ("rope_step", time_rope_step), ("prefill", time_prefill)):
        if name in wanted:
            also[name] = fn(ada, device)
    if not args.no_cpu_baseline and not args.long_context_only:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
