"""Benchmark of the single-token decode-attention hot path on one MI355X.

A step is one pass of the whole hot path over the one-token MHA decode sweep
of Cuda-Compute-OSS #343 ("Current limitation"): batch 1, 16 query heads = 16
KV heads, head_dim 128, fp16, capacity 8192; for each kv_len in
(1024, 4096, 8192): append the new K/V rows at slot kv_len - 1, then decode
over kv_len slots. Each kv_len has its own cache, and steps rotate over 5 sets
of caches (960 MiB) so that no call finds its K/V in the 256 MB Infinity Cache:
the inputs sit in HBM when the timed region starts.

The timed region replays one HIP graph per step (the step's 9 kernels:
3 x append, partial, combine); eager launches from Python are reported
beside it. Printed: one JSON line with the metric (achieved algorithmic GB/s
over the timed steps), the roofline of the dominant kernel (the split-KV
partial: algorithmic bytes / its average duration over back-to-back launches
bracketed by HIP events, with the host queued ahead so that launch cost does
not count, against 8 TB/s), the fp64 CPU oracle timed on a bounded sample of
the same step, and, under "also", the per-kv_len figures, the
long-context workload (batch 8, 32/8 heads, bf16, kv_len 32768, 1.07 GB per
call), the 36-layer S2-Pro-shaped run, the MiniCPM-shaped streaming
workload (lockstep positions and ragged batches), the full-capacity against
active-prefix comparison, the decode step with rotary embedding, and the
causal prompt prefill.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
PMC_SUMMARY = ROOT / "profiles" / "decode_kernel_mha_sweep_pmc.md"


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
    """HBM bytes of one step's partial-kernel launches from the committed
    rocprofv3 counter summary, or None when there is none or the kernel source
    changed since the counters were taken."""
    if not PMC_SUMMARY.exists():
        return None
    text = PMC_SUMMARY.read_text()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_step_decode:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


# ---------------------------------------------------------------------------


class Sweep:
    """The one-token MHA decode sweep with rotating cold caches."""

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
        self.k_new, self.v_new = W.append_inputs(B, Hkv, D, shp.dtype, W.seed_for(1, 9000), device=device)
        self.pos = [torch.full((B,), n - 1, dtype=torch.int32, device=device) for n in SWEEP]
        self.lens = [torch.full((B,), n, dtype=torch.int32, device=device) for n in SWEEP]
        self.out = [torch.empty((B, Hq, D), dtype=W.TORCH_DTYPES[shp.dtype], device=device) for _ in SWEEP]
        self.scale = 1.0 / math.sqrt(D)
        self.decode_bytes = [decode_bytes(B, Hq, Hkv, D, [n]) for n in SWEEP]
        self.step_bytes = sum(self.decode_bytes) + 3 * append_bytes(B, Hkv, D)
        self.i = 0
        ws_need = max(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, ada.decode_num_splits(B, Hq, Hkv, n)))
                      for n in SWEEP)
        self.ws = ada.new_workspace(ws_need, device)

    def step(self, set_index: int | None = None):
        """One decode step at each kv_len -- append the new row at slot kv_len - 1
        and attend over kv_len slots, as one ada_decode_step call (partial
        kernel with the append folded in, then the combine kernel) -- on the
        next cache set (or ``set_index``). The position is a host int (batch
        1), so the kernels read no length from the device."""
        ada = self.ada
        row = self.caches[(self.i if set_index is None else set_index) % self.sets]
        self.i += 1
        for j, n in enumerate(SWEEP):
            k, v = row[j]
            ada.decode_step(self.q[j], self.k_new, self.v_new, k, v, n - 1, scale=self.scale, out=self.out[j],
                            workspace=self.ws)

    def capture(self):
        """One HIP graph per cache set holding a whole step (6 kernels)."""
        self.graphs = []
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for s in range(self.sets):  # warm the binding's caches outside capture
                self.step(s)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        for s in range(self.sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(s)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay(self):
        self.graphs[self.i % self.sets].replay()
        self.i += 1

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


def time_long_context(ada, device, iters: int = 20) -> dict:
    """The long-context workload (1.07 GB per call, 4x the Infinity Cache, so
    every call streams from HBM): average partial-kernel and whole-call
    durations over back-to-back launches bracketed by HIP events."""
    wl = W.WORKLOADS["long_context"]
    shp = wl.shape
    x = W.decode_inputs(shp, [shp.capacity] * shp.batch, W.seed_for(4), device=device, tail="random",
                        outlier_p=wl.outlier_p, outlier_scale=wl.outlier_scale)
    B, Hq, Hkv, D = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim
    splits = ada.decode_num_splits(B, Hq, Hkv, shp.capacity)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, splits)), device)
    out = torch.empty_like(x["q"])
    scale = 1.0 / math.sqrt(D)

    def partial():
        return ada.decode_partial(x["q"], x["k_cache"], x["v_cache"], None, scale=scale,
                                  max_kv_len=shp.capacity, workspace=ws)[1]

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    for _ in range(3):
        ada.decode_combine(ws, partial(), out, Hkv)
    part = timed(partial)
    whole = timed(lambda: ada.decode_combine(ws, partial(), out, Hkv))
    nbytes = decode_bytes(B, Hq, Hkv, D, [shp.capacity] * B)
    del x
    return {"workload": "long_context: batch 8, 32/8 heads, head_dim 128, bf16, kv_len 32768, 1% keys x8",
            "bytes_per_call": nbytes, "splits": splits,
            "partial_us": round(part, 2), "partial_GBs": round(nbytes / part / 1e3, 1),
            "partial_frac_of_peak": round(nbytes / part / 1e3 / PEAK_HBM_GBS, 4),
            "call_us": round(whole, 2), "call_GBs": round(nbytes / whole / 1e3, 1),
            "call_frac_of_peak": round(nbytes / whole / 1e3 / PEAK_HBM_GBS, 4)}


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
        res[f"lockstep_p{p}"] = {"us": round(us, 2), "GBs": round(nb / us / 1e3, 1),
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
    res["ragged"] = {"draws": draws, "mean_us": round(tot_us / draws, 2), "GBs": round(tot_b / tot_us / 1e3, 1),
                     "frac_of_peak": round(tot_b / tot_us / 1e3 / PEAK_HBM_GBS, 4),
                     "draws_mean_len_ge_4096": len(big),
                     "GBs_mean_len_ge_4096": round(sum(r[2] for r in big) / max(1e-9, sum(r[1] for r in big)) / 1e3, 1)}
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


def cpu_baseline(seconds: float) -> dict:
    """The fp64 oracle on the same step (three decode calls of the sweep), run
    until ``seconds`` of CPU time have passed (at least one step)."""
    import oracle

    ora = oracle.load()
    shp = W.WORKLOADS["mha_sweep"].shape
    B, Hq, Hkv, D = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim
    inputs = []
    for j, n in enumerate(SWEEP):
        x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, n, shp.dtype), [n], W.seed_for(1, j), tail="random")
        inputs.append((x, n))
    scale = 1.0 / math.sqrt(D)
    steps = 0
    t0 = time.perf_counter()
    while True:
        for x, n in inputs:
            ora.decode(x["q"], x["k_cache"], x["v_cache"], [n], scale)
        steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    nbytes = steps * sum(decode_bytes(B, Hq, Hkv, D, [n]) for n in SWEEP)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": ora.threads(), "kind": "oracle",
            "sample": f"{steps} steps of the MHA sweep decode calls (kv_len 1024/4096/8192, batch 1, 16 heads, "
                      f"fp16) in {dt:.1f} s; cache appends not included",
            "ms_per_step": round(dt / steps * 1e3, 2)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-long-context", action="store_true")
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
    if args.prefill_only:
        print(json.dumps({"prefill": time_prefill(ada, device)}), flush=True)
        return 0
    torch.cuda.set_device(device)
    # A plain copy of known size (256 MiB read, 256 MiB written): the reference
    # that scales the FETCH_SIZE / WRITE_SIZE counters of the profiled runs.
    calib_src = torch.empty(CALIB_BYTES // 2, dtype=torch.float16, device=device).fill_(1.0)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    sweep = Sweep(ada, device)
    launch = "hip_graph"
    try:
        sweep.capture()
    except Exception as exc:  # graph capture unavailable: time eager launches instead
        launch = f"eager ({type(exc).__name__})"
        sweep.graphs = None
    run_step = sweep.replay if sweep.graphs else sweep.step
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = sweep.step_bytes / (ms_per_step * 1e-3) / 1e9

    # Eager steps (every kernel launched from Python through the C ABI).
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for _ in range(args.steps):
        sweep.step()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - e0) * 1e3 / args.steps

    part_us = sweep.time_partials(args.steps)
    call_us = sweep.time_calls(args.steps)
    hot_us = sweep.time_calls(args.steps, resident=True)
    per_kv = []
    for j, n in enumerate(SWEEP):
        nb = sweep.decode_bytes[j]
        per_kv.append({"kv_len": n, "bytes": nb, "splits": ada.decode_num_splits(1, 16, 16, n),
                       "partial_us": round(part_us[j], 2), "partial_GBs": round(nb / part_us[j] / 1e3, 1),
                       "call_us": round(call_us[j], 2), "call_GBs": round(nb / call_us[j] / 1e3, 1),
                       "call_frac_of_peak": round(nb / call_us[j] / 1e3 / PEAK_HBM_GBS, 4),
                       "cache_resident_call_us": round(hot_us[j], 2),
                       "cache_resident_call_GBs": round(nb / hot_us[j] / 1e3, 1)})
    achieved = sum(sweep.decode_bytes) / sum(part_us) / 1e3
    traffic = pmc_traffic()

    also = {"per_kv_len": per_kv, "eager_ms_per_step": round(eager_ms, 4),
            "eager_GBs": round(sweep.step_bytes / (eager_ms * 1e-3) / 1e9, 1)}
    if not args.no_long_context:
        also["long_context"] = time_long_context(ada, device)
        also["shards"] = time_shards(ada, device)
        also["s2pro_run"] = time_s2pro_run(ada, device)
        also["full_capacity_vs_active_prefix"] = time_full_vs_active(ada, device)
        also["minicpm_stream"] = time_minicpm_stream(ada, device)
        also["minicpm_sweep"] = time_minicpm_sweep(ada, device)
        also["rope_step"] = time_rope_step(ada, device)
        also["prefill"] = time_prefill(ada, device)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "mha_sweep: one-token decode, batch 1, 16 heads = 16 KV heads, head_dim 128, fp16, "
                               "kv_len 1024/4096/8192 (append + decode each), capacity 8192, "
                               f"cold caches rotated over {sweep.sets} sets",
                   "step_bytes": sweep.step_bytes, "kernels_per_step": 6, "launch": launch},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "traffic_basis": "HBM bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of the three partial "
                                      "launches of one step; algorithmic bytes of the same launches: "
                                      f"{sum(sweep.decode_bytes)}",
                     "kernel": "partial_kernel (split-KV partial of the decode; the combine kernel follows it)",
                     "bytes_per_launch": sweep.decode_bytes,
                     "us_per_launch": [round(u, 2) for u in part_us]},
        "also": also,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
