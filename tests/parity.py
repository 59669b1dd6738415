"""Comparison of GPU outputs against the oracle (float64), shared by the GPU
tests, the smoke check and the benchmark.

Tolerances: max-abs 4e-3 / relative Frobenius 1e-3 for fp16 outputs, 1.6e-2 /
4e-3 for bf16 outputs, over the whole output tensor of a call, and every
output finite. They are tighter than the bar the one-token decode fast-path
page sets (relative Frobenius 0.005, abs 0.05; Cuda-Compute-OSS #343,
"Expected measurement") and sit above what fp32 accumulation plus one
round-to-nearest-even output rounding can cost: half an ulp of an output below
8 in magnitude is at most 2e-3 in fp16 and 7.8e-3 in bf16 (below 4).
The prompt prefill, whose softmax weights are rounded to 16 bits for the
matrix cores, is checked against a per-element bound derived from that
arithmetic instead of the fixed max-abs (prefill_bound below).
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


# Prompt prefill: the softmax weights enter the matrix-core product P.V
# rounded once to the 16-bit type of the cache (unit roundoff u = 2^-11 for
# fp16, 2^-8 for bf16), numerator and denominator alike. With w_j the exact
# weights and w_j (1 + d_j), |d_j| <= u, the rounded ones, the normalised sum
# moves by sum_j w_j d_j (v_j - o) / sum_j w_j (1 + d_j), at most
# u / (1 - u) * max_j |v_j - o| over the visible slots j; the output rounding
# then adds half an ulp of the result. The fp32 sums (the value products on
# the matrix cores, n / 32 accumulations per output for n visible slots; the
# row sum, at most n / 8 per lane plus the cross-lane adds; the final
# division) add at most (n / 8 + 16) * 2^-24 * (max_j |v_j| + |o|). This
# per-element bound replaces the fixed max-abs for the prefill (an output
# near a bf16 binade top of 4 or 8 already spends a whole half ulp, 7.8e-3 or
# 1.6e-2, on the final rounding); the relative Frobenius tolerance stays as
# above.
UNIT_ROUNDOFF = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
SIGNIFICAND_BITS = {"fp16": 11, "bf16": 8}
SUBNORMAL_HALF_ULP = {"fp16": 2.0 ** -25, "bf16": 2.0 ** -134}  # below the normal range the ulp is fixed


def prefill_bound(want: np.ndarray, v: torch.Tensor, lens, dtype: str) -> np.ndarray:
    """Per-element error bound for prefill outputs ``want`` [B, H_q, T', D]
    (the oracle's), given the value cache ``v`` [B, H_kv, S, D] and ``lens``
    [B, T'] the visible slot count of each output token (0: the output is an
    exact zero)."""
    vv = v.detach().to("cpu").to(torch.float64).numpy()
    B, Hq, Tn, D = want.shape
    G = Hq // vv.shape[1]
    lens = np.asarray(lens, dtype=np.int64).reshape(B, Tn)
    u = UNIT_ROUNDOFF[dtype]
    p = SIGNIFICAND_BITS[dtype]
    bound = np.zeros_like(want)
    for b in range(B):
        live = lens[b] > 0
        idx = np.maximum(lens[b] - 1, 0)
        for g in range(vv.shape[1]):
            top = np.maximum.accumulate(vv[b, g], axis=0)[idx]  # [T', D]: max of v over the visible slots
            bot = np.minimum.accumulate(vv[b, g], axis=0)[idx]
            n = lens[b].astype(np.float64)[:, None]
            for h in range(g * G, (g + 1) * G):
                o = want[b, h]
                spread = np.maximum(top - o, o - bot)
                w = u / (1.0 - u) * spread
                sums = (n / 8 + 16) * 2.0 ** -24 * (np.maximum(np.abs(top), np.abs(bot)) + np.abs(o))
                mag = np.maximum(np.abs(o) + w + sums, 2.0 ** -126)
                half_ulp = np.maximum(2.0 ** (np.floor(np.log2(mag)) - p), SUBNORMAL_HALF_ULP[dtype])
                bound[b, h] = np.where(live[:, None], half_ulp + w + sums, 0.0)
    return bound


def assert_parity_bound(got: torch.Tensor, want: np.ndarray, bound: np.ndarray, dtype: str, what: str = "") -> dict:
    """Finite outputs, |got - want| <= bound element by element, and the
    relative Frobenius tolerance of the dtype."""
    st = compare(got, want)
    g = to_f64(got).reshape(want.shape)
    ratio = float(np.max(np.abs(g - want) / np.maximum(bound, 1e-300))) if g.size else 0.0
    rel = TOL[dtype][1]
    print(f"  parity {what}: max-abs {st['max_abs']:.2e} (largest error / bound {ratio:.2f}), "
          f"rel-Frobenius {st['rel_fro']:.2e} (tol {rel:.1e})", flush=True)
    assert st["finite"], f"{what}: non-finite GPU output"
    bad = np.abs(g - want) > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs beyond the per-element bound "
                           f"(largest error / bound {ratio:.3f})")
    assert st["rel_fro"] <= rel, f"{what}: rel-Frobenius {st['rel_fro']:.3e} > {rel:.1e}"
    return st
