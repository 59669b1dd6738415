"""Benchmark of the single-token decode-attention hot path on one MI355X.

A step is one pass of the whole hot path over the one-token MHA decode sweep
of Cuda-Compute-OSS #343 ("Current limitation"): batch 1, 16 query heads = 16
KV heads, head_dim 128, fp16, capacity 8192; for each kv_len in
(1024, 4096, 8192): append the new K/V rows at slot kv_len - 1, then decode
over kv_len slots. Each kv_len has its own cache, and steps rotate over 5 sets
of caches (960 MiB) so that no call finds its K/V in the 256 MB Infinity Cache:
the inputs sit in HBM when the timed region starts.

Printed: one JSON line with the metric (achieved algorithmic GB/s over the
timed steps), the decode kernel's roofline (algorithmic bytes / its average
duration from HIP events around each launch, against 8 TB/s), the fp64 CPU
oracle timed on a bounded sample of the same step, and, under "also", the
per-kv_len figures and the long-context workload (batch 8, 32/8 heads, bf16,
kv_len 32768, 1.07 GB per call).

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


def pmc_traffic(bytes_key: str = "mha_sweep") -> float | None:
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since it was taken."""
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
        ws_need = max(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, ada.decode_num_splits(B, Hkv, n)))
                      for n in SWEEP)
        self.ws = ada.new_workspace(ws_need, device)

    def step(self, events=None):
        """Append then decode at each kv_len; the decode is issued as its two
        kernels (partial, combine) so that HIP events bracket the partial
        kernel alone: events[j] = (before partial, after partial, after combine)."""
        ada = self.ada
        row = self.caches[self.i % self.sets]
        self.i += 1
        for j, n in enumerate(SWEEP):
            k, v = row[j]
            ada.kv_append(self.k_new, self.v_new, k, v, self.pos[j])
            if events is not None:
                events[j][0].record()
            _, used = ada.decode_partial(self.q[j], k, v, self.lens[j], scale=self.scale, max_kv_len=n,
                                         workspace=self.ws)
            if events is not None:
                events[j][1].record()
            ada.decode_combine(self.ws, used, self.out[j], self.shape.n_kv_head)
            if events is not None:
                events[j][2].record()
        self.splits = used


def time_long_context(ada, device, iters: int = 20) -> dict:
    """The long-context workload (1.07 GB per call, 4x the Infinity Cache, so
    every call streams from HBM): HIP events around each partial kernel and
    around each whole call (partial + combine)."""
    wl = W.WORKLOADS["long_context"]
    shp = wl.shape
    x = W.decode_inputs(shp, [shp.capacity] * shp.batch, W.seed_for(4), device=device, tail="random",
                        outlier_p=wl.outlier_p, outlier_scale=wl.outlier_scale)
    B, Hq, Hkv, D = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim
    splits = ada.decode_num_splits(B, Hkv, shp.capacity)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, splits)), device)
    out = torch.empty_like(x["q"])
    scale = 1.0 / math.sqrt(D)

    def call(ev=None):
        if ev:
            ev[0].record()
        _, used = ada.decode_partial(x["q"], x["k_cache"], x["v_cache"], x["kv_len"], scale=scale,
                                     max_kv_len=shp.capacity, workspace=ws)
        if ev:
            ev[1].record()
        ada.decode_combine(ws, used, out, Hkv)
        if ev:
            ev[2].record()

    for _ in range(5):
        call()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(iters)]
    torch.cuda.synchronize()
    for ev in evs:
        call(ev)
    torch.cuda.synchronize()
    part = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in evs)
    whole = sorted(e[0].elapsed_time(e[2]) * 1e3 for e in evs)
    nbytes = decode_bytes(B, Hq, Hkv, D, [shp.capacity] * B)
    med = lambda v: v[len(v) // 2]
    del x
    return {"workload": "long_context: batch 8, 32/8 heads, head_dim 128, bf16, kv_len 32768, 1% keys x8",
            "bytes_per_call": nbytes, "splits": splits,
            "partial_us_median": round(med(part), 2), "partial_GBs": round(nbytes / med(part) / 1e3, 1),
            "partial_frac_of_peak": round(nbytes / med(part) / 1e3 / PEAK_HBM_GBS, 4),
            "call_us_median": round(med(whole), 2), "call_GBs": round(nbytes / med(whole) / 1e3, 1),
            "call_frac_of_peak": round(nbytes / med(whole) / 1e3 / PEAK_HBM_GBS, 4)}


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
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode kernel needs no exchange between GPUs "
              "(batch rows and KV heads are independent); run with --gpus 1.", file=sys.stderr)
        return 2

    import autoregressive_decode_attention_amd as ada

    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    sweep = Sweep(ada, device)
    for _ in range(args.warmup):
        sweep.step()
    events = [[tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in SWEEP]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        sweep.step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = sweep.step_bytes / (ms_per_step * 1e-3) / 1e9

    per_kv = []
    part_us_total = 0.0
    part_bytes_total = 0
    for j, n in enumerate(SWEEP):
        part = [events[k][j][0].elapsed_time(events[k][j][1]) * 1e3 for k in range(args.steps)]
        whole = [events[k][j][0].elapsed_time(events[k][j][2]) * 1e3 for k in range(args.steps)]
        pm, wm = sum(part) / len(part), sum(whole) / len(whole)
        part_us_total += pm
        part_bytes_total += sweep.decode_bytes[j]
        nb = sweep.decode_bytes[j]
        per_kv.append({"kv_len": n, "bytes": nb, "splits": ada.decode_num_splits(1, 16, n),
                       "partial_us_mean": round(pm, 2), "partial_GBs": round(nb / pm / 1e3, 1),
                       "call_us_mean": round(wm, 2), "call_us_median": round(sorted(whole)[len(whole) // 2], 2),
                       "call_GBs": round(nb / wm / 1e3, 1), "call_frac_of_peak": round(nb / wm / 1e3 / PEAK_HBM_GBS, 4)})
    achieved = part_bytes_total / part_us_total / 1e3
    traffic = pmc_traffic()

    also = {"per_kv_len": per_kv}
    if not args.no_long_context:
        also["long_context"] = time_long_context(ada, device)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "mha_sweep: one-token decode, batch 1, 16 heads = 16 KV heads, head_dim 128, fp16, "
                               "kv_len 1024/4096/8192 (append + decode each), capacity 8192, "
                               f"cold caches rotated over {sweep.sets} sets",
                   "step_bytes": sweep.step_bytes, "calls_per_step": 6},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "partial_kernel (split-KV partial of the decode; the combine kernel follows it)",
                     "bytes_per_launch": sweep.decode_bytes,
                     "us_per_launch": [p["partial_us_mean"] for p in per_kv]},
        "also": also,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
