"""Comparison of GPU outputs against the oracle (float64), shared by the GPU
tests, the smoke check and the benchmark.

Tolerances: max-abs 4e-3 / relative Frobenius 1e-3 for fp16 outputs, 1.6e-2 /
4e-3 for bf16 outputs, over the whole output tensor of a call, and every
output finite. They are tighter than the bar the one-token decode fast-path
page sets (relative Frobenius 0.005, abs 0.05; Cuda-Compute-OSS #343,
"Expected measurement") and sit above what fp32 accumulation plus one
round-to-nearest-even output rounding can cost: half an ulp of an output below
8 in magnitude is at most 2e-3 in fp16 and 7.8e-3 in bf16 (below 4).
The prompt prefill is held to the same tolerances.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"fp16": (4e-3, 1e-3), "bf16": (1.6e-2, 4e-3)}


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def compare(got: torch.Tensor, want: np.ndarray) -> dict:
    g = to_f64(got).reshape(want.shape)
    diff = g - want
    ref = float(np.linalg.norm(want))
    return {
        "finite": bool(np.all(np.isfinite(g))),
        "max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "rel_fro": float(np.linalg.norm(diff) / ref) if ref > 0 else float(np.linalg.norm(diff)),
    }


def assert_parity(got: torch.Tensor, want: np.ndarray, dtype: str, what: str = "") -> dict:
    st = compare(got, want)
    max_abs, rel = TOL[dtype]
    print(f"  parity {what}: max-abs {st['max_abs']:.2e} (tol {max_abs:.1e}), rel-Frobenius {st['rel_fro']:.2e} "
          f"(tol {rel:.1e})", flush=True)
    assert st["finite"], f"{what}: non-finite GPU output"
    assert st["max_abs"] <= max_abs, f"{what}: max-abs {st['max_abs']:.3e} > {max_abs:.1e}"
    assert st["rel_fro"] <= rel, f"{what}: rel-Frobenius {st['rel_fro']:.3e} > {rel:.1e}"
    return st

