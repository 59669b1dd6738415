"""Seeded synthetic inputs for single-token decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Both sides of every parity check (the CPU oracle and the
GPU library) and the benchmark take their inputs from here, so that neither
side depends on the other.

Workload shapes follow the pages (cited by title and section):

* ``tiny``: one layer of the fish-speech S2-Pro attention shape (32 query
  heads sharing 8 KV heads, head_dim 128; fish-speech issue #1310 "Optimize
  native AR decoding by attending only to the active KV-cache prefix",
  section 1), fp16, 400 live slots in a 2048-slot cache.
* ``mha_sweep``: the three one-token decode workloads of Cuda-Compute-OSS
  issue #343 ("one-token decode fast path ..."), section "Current
  limitation": batch 1, 16 heads, head_dim 128, fp16, kv_len 1024/4096/8192.
* ``s2pro_run``: the S2-Pro decode run of fish-speech issue #1310, "CUDA
  benchmark" (36 layers, capacity 32768, a 234-token prompt, 1024 new
  tokens), fp16.
* ``minicpm_stream``: the MiniCPM4 forward_step cache of VoxCPM issue #395,
  section 2.2 (batch, 8 KV heads, 8192 slots, head_dim 128) with 32 query
  heads, bf16, batch 4, positions swept 0..8191 and ragged per-row lengths.
* ``long_context``: batch 8, 32/8 heads, bf16, 32768 live slots, with 1% of
  key rows scaled by 8 to widen the score range.

Values are N(0, 1) drawn in float32 from a seeded ``torch.Generator`` and
rounded to the 16-bit type by round-to-nearest-even. Seed ``42 + c`` for
configuration ``c`` (42 is the seed of the S2-Pro run), sub-stream
``(42 + c) * 1_000_003 + k`` for layer, step or draw ``k``. Cache slots at and
beyond a row's kv_len are filled with NaN in parity runs (they must never be
read) and left random or zero otherwise.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

TORCH_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class DecodeShape:
    batch: int
    n_head: int
    n_kv_head: int
    head_dim: int
    capacity: int
    dtype: str


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    shape: DecodeShape
    kv_lens: tuple = ()
    layers: int = 1
    prefill: int = 0
    steps: int = 0
    outlier_p: float = 0.0
    outlier_scale: float = 8.0
    notes: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 0, DecodeShape(1, 32, 8, 128, 2048, "fp16"), kv_lens=(400,)),
    "mha_sweep": Workload("mha_sweep", 1, DecodeShape(1, 16, 16, 128, 8192, "fp16"),
                          kv_lens=(1024, 4096, 8192)),
    "s2pro_run": Workload("s2pro_run", 2, DecodeShape(1, 32, 8, 128, 32768, "fp16"),
                          layers=36, prefill=234, steps=1024),
    "minicpm_stream": Workload("minicpm_stream", 3, DecodeShape(4, 32, 8, 128, 8192, "bf16"),
                               steps=8192),
    "long_context": Workload("long_context", 4, DecodeShape(8, 32, 8, 128, 32768, "bf16"),
                             kv_lens=(32768,), outlier_p=0.01, outlier_scale=8.0),
}


def seed_for(index: int, k: int | None = None) -> int:
    base = 42 + index
    return base if k is None else base * 1_000_003 + k


def _generator(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev.type if dev.type != "cuda" else dev)
    g.manual_seed(seed)
    return g


def randn16(shape, dtype: str, seed: int, device="cpu") -> torch.Tensor:
    """N(0, 1) in float32, rounded to the 16-bit type (round-to-nearest-even)."""
    g = _generator(seed, device)
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(TORCH_DTYPES[dtype])


def decode_inputs(shape: DecodeShape, kv_len, seed: int, *, device="cpu", tail: str = "nan",
                  outlier_p: float = 0.0, outlier_scale: float = 8.0) -> dict:
    """q [B, Hq, D], k_cache and v_cache [B, Hkv, S, D], kv_len int32 [B].

    ``tail`` fills slots ``j >= kv_len[b]``: "nan", "zero" or "random" (keep
    the drawn values). With ``outlier_p > 0`` a seeded Bernoulli mask over
    (batch, KV head, slot) scales whole key rows by ``outlier_scale`` before
    rounding (a power of two, so the scaling itself is exact).
    """
    B, Hq, Hkv, D, S = shape.batch, shape.n_head, shape.n_kv_head, shape.head_dim, shape.capacity
    lens = [int(x) for x in (kv_len if hasattr(kv_len, "__len__") else [kv_len] * B)]
    if len(lens) != B:
        raise ValueError("kv_len must have one entry per batch row")
    g = _generator(seed, device)
    f32 = dict(generator=g, dtype=torch.float32, device=device)
    dt = TORCH_DTYPES[shape.dtype]
    q = torch.randn((B, Hq, D), **f32).to(dt)
    k = torch.randn((B, Hkv, S, D), **f32)
    if outlier_p > 0.0:
        mask = torch.rand((B, Hkv, S, 1), **f32) < outlier_p
        k = torch.where(mask, k * outlier_scale, k)
        del mask
    k = k.to(dt)
    v = torch.randn((B, Hkv, S, D), **f32).to(dt)
    if tail != "random":
        fill = float("nan") if tail == "nan" else 0.0
        for b, n in enumerate(lens):
            n = max(0, min(n, S))
            k[b, :, n:, :] = fill
            v[b, :, n:, :] = fill
    lens_t = torch.tensor(lens, dtype=torch.int32, device=device)
    return {"q": q, "k_cache": k, "v_cache": v, "kv_len": lens_t}


def append_inputs(batch: int, n_kv_head: int, head_dim: int, dtype: str, seed: int, device="cpu"):
    """New key and value rows [B, Hkv, D] for one cache append."""
    g = _generator(seed, device)
    f32 = dict(generator=g, dtype=torch.float32, device=device)
    dt = TORCH_DTYPES[dtype]
    k_new = torch.randn((batch, n_kv_head, head_dim), **f32).to(dt)
    v_new = torch.randn((batch, n_kv_head, head_dim), **f32).to(dt)
    return k_new, v_new


def rope_tables(positions, head_dim: int, dtype: str, base: float = 10000.0, device="cpu"):
    """cos / sin rows [B, D] for the given per-row positions, rotate-half layout.

    Angles pos * base^(-2i/D) for i < D/2, repeated in both halves (the usual
    rotary frequencies; the pages do not give the model's own, so these are a
    synthetic stand-in), evaluated in float64 and rounded to the 16-bit dtype.
    """
    pos = torch.as_tensor(positions, dtype=torch.float64).reshape(-1, 1)
    inv = base ** (-torch.arange(0, head_dim, 2, dtype=torch.float64) / head_dim)
    theta = torch.cat([pos * inv, pos * inv], dim=1)
    dt = TORCH_DTYPES[dtype]
    return torch.cos(theta).to(dt).to(device), torch.sin(theta).to(dt).to(device)


def ragged_lengths(batch: int, low: int, high: int, seed: int) -> list:
    """Per-row kv_len drawn uniformly from [low, high], seeded."""
    g = torch.Generator().manual_seed(seed)
    return [int(x) for x in torch.randint(low, high + 1, (batch,), generator=g)]
