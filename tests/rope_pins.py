"""Pins for the rotary oracle (``oracle/rope.py``), each reached another way.

Every pin takes the module under test (the real oracle, or a mutated copy in
``test_rope_oracle.py``) and raises AssertionError when it disagrees with:

- exact identities of the map (cos = 1, sin = 0 is the identity; cos = 0,
  sin = 1 is the quarter turn that moves each half onto the other with the
  first half negated; cos = -1, sin = 0 negates);
- complex multiplication of the pairs (x[i] + i x[i+h]) by (cos + i sin) in
  numpy complex128, converted by numpy's own float64 -> float16 rounding;
- the rotate-half operator written as an explicit D x D signed permutation
  matrix, applied with numpy matmul (general cos/sin rows whose halves
  differ), again converted by numpy;
- hand-built halfway cases whose rounding the format fixes (ties to the even
  pattern, and the overflow threshold halfway past the largest value);
- the relative-position property of rotary embeddings: with tables built
  from angles pos * theta_i, the score of a query rotated at position a
  with a key rotated at position b depends only on a - b;
- locality: output i depends only on inputs i and i +- h.

Inputs of the numpy comparisons keep every product within a few binades of
the others, so the float64 arithmetic on the way is exact and numpy's single
rounding is the correctly rounded result.
"""
from __future__ import annotations

import math

import numpy as np
import torch

ONE = {"fp16": 0x3C00, "bf16": 0x3F80}
NEG_ONE = {"fp16": 0xBC00, "bf16": 0xBF80}
INF = {"fp16": 0x7C00, "bf16": 0x7F80}
TORCH = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _randn_bits(shape, fmt, seed, lo=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if lo is not None:  # keep magnitudes in [lo, 4) so products stay within a few binades
        x = torch.sign(x) * x.abs().clamp(lo, 3.9)
        x[x == 0] = lo
    return _bits(x.to(TORCH[fmt]))


def _const(shape, bits):
    return np.full(shape, bits, dtype=np.uint16)


def _f64(bits, fmt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH[fmt])
    return t.to(torch.float64).numpy()


def pin_identity(mod):
    for fmt in ("fp16", "bf16"):
        x = _randn_bits((2, 3, 16), fmt, 11)
        x[0, 0, 5] = 0x8000  # -0 comes back as +0
        out = mod.rope(x, _const((2, 16), ONE[fmt]), _const((2, 16), 0), fmt)
        want = x.copy()
        want[0, 0, 5] = 0
        assert np.array_equal(out, want), f"{fmt}: cos = 1, sin = 0 must return the input"


def pin_quarter_turn(mod):
    for fmt in ("fp16", "bf16"):
        x = _randn_bits((2, 2, 16), fmt, 12)
        out = mod.rope(x, _const((2, 16), 0), _const((2, 16), ONE[fmt]), fmt)
        h = 8
        want = np.concatenate([x[..., h:] ^ 0x8000, x[..., :h]], axis=-1).astype(np.uint16)
        assert np.array_equal(out, want), f"{fmt}: cos = 0, sin = 1 must map (a, b) to (-b, a)"


def pin_half_turn(mod):
    for fmt in ("fp16", "bf16"):
        x = _randn_bits((1, 3, 16), fmt, 13)
        out = mod.rope(x, _const((1, 16), NEG_ONE[fmt]), _const((1, 16), 0), fmt)
        assert np.array_equal(out, x ^ 0x8000), f"{fmt}: cos = -1, sin = 0 must negate"


def _angle_tables(batch, d, fmt, seed):
    """cos/sin rows from random angles with |cos|, |sin| in [0.5, 1] (same angle in both halves)."""
    g = np.random.default_rng(seed)
    h = d // 2
    quad = g.integers(0, 4, size=(batch, h))
    theta = quad * (math.pi / 2) + g.uniform(math.pi / 6, math.pi / 3, size=(batch, h))
    theta = np.concatenate([theta, theta], axis=1)
    c = _bits(torch.from_numpy(np.cos(theta)).to(TORCH[fmt]))
    s = _bits(torch.from_numpy(np.sin(theta)).to(TORCH[fmt]))
    return c, s


def pin_complex_multiply(mod):
    fmt = "fp16"
    d, h = 32, 16
    x = _randn_bits((3, 4, d), fmt, 14, lo=0.5)
    c, s = _angle_tables(3, d, fmt, 15)
    out = mod.rope(x, c, s, fmt)
    xf, cf, sf = _f64(x, fmt), _f64(c, fmt), _f64(s, fmt)
    z = (xf[..., :h] + 1j * xf[..., h:]) * (cf[:, None, :h] + 1j * sf[:, None, :h])
    want = np.concatenate([z.real, z.imag], axis=-1).astype(np.float16).view(np.uint16)
    assert np.array_equal(out, want), "rotation differs from complex multiplication of the pairs"


def pin_operator_matrix(mod):
    fmt = "fp16"
    d, h = 16, 8
    x = _randn_bits((2, 3, d), fmt, 16, lo=0.5)
    g = np.random.default_rng(17)
    # general rows: the two halves carry different angles
    theta = g.uniform(math.pi / 6, math.pi / 3, size=(2, d)) + g.integers(0, 4, size=(2, d)) * (math.pi / 2)
    c = _bits(torch.from_numpy(np.cos(theta)).to(torch.float16))
    s = _bits(torch.from_numpy(np.sin(theta)).to(torch.float16))
    out = mod.rope(x, c, s, fmt)
    # rotate_half(x) = P @ x with P[i, i + h] = -1 (i < h) and P[i, i - h] = +1 (i >= h)
    P = np.zeros((d, d))
    for i in range(h):
        P[i, i + h] = -1.0
        P[i + h, i] = 1.0
    xf, cf, sf = _f64(x, fmt), _f64(c, fmt), _f64(s, fmt)
    want = xf * cf[:, None, :] + np.einsum("ij,bhj->bhi", P, xf) * sf[:, None, :]
    want = want.astype(np.float16).view(np.uint16)
    assert np.array_equal(out, want), "rotation differs from x * cos + rotate_half(x) * sin"


def pin_bf16_exact_sums(mod):
    """bf16 results that are exact in float32 are rounded once by torch's float32 -> bf16 conversion."""
    fmt = "bf16"
    d, h = 16, 8
    x = _randn_bits((2, 3, d), fmt, 18, lo=0.5)
    c, s = _angle_tables(2, d, fmt, 19)
    out = mod.rope(x, c, s, fmt)
    xf, cf, sf = _f64(x, fmt), _f64(c, fmt), _f64(s, fmt)
    z = (xf[..., :h] + 1j * xf[..., h:]) * (cf[:, None, :h] + 1j * sf[:, None, :h])
    exact = np.concatenate([z.real, z.imag], axis=-1)
    as32 = exact.astype(np.float32)
    assert np.array_equal(as32.astype(np.float64), exact), "test inputs must give float32-exact sums"
    want = _bits(torch.from_numpy(as32).to(torch.bfloat16))
    assert np.array_equal(out, want), "bf16 rotation differs from the correctly rounded sums"


def _one_pair(mod, fmt, a, b, c, s):
    """Rotate a single pair (a, b) with tables c, s (bit patterns); returns (out0, out1)."""
    x = np.array([[[a, b]]], dtype=np.uint16)
    cc = np.array([[c, c]], dtype=np.uint16)
    ss = np.array([[s, s]], dtype=np.uint16)
    out = mod.rope(x, cc, ss, fmt)
    return int(out[0, 0, 0]), int(out[0, 0, 1])


def pin_rounding_ties(mod):
    # fp16: second output = b * 1 + a * 1 with a = 2^-11 (half an ulp of values in [1, 2))
    half_ulp = 0x1000  # 2^-11
    assert _one_pair(mod, "fp16", half_ulp, 0x3C01, ONE["fp16"], ONE["fp16"])[1] == 0x3C02  # odd -> up
    assert _one_pair(mod, "fp16", half_ulp, 0x3C02, ONE["fp16"], ONE["fp16"])[1] == 0x3C02  # even stays
    assert _one_pair(mod, "fp16", half_ulp ^ 0x8000, 0xBC01, ONE["fp16"], ONE["fp16"])[1] == 0xBC02
    assert _one_pair(mod, "fp16", 0x0C00, 0x3C02, ONE["fp16"], ONE["fp16"])[1] == 0x3C02  # 2^-12: below half
    # bf16: a = 2^-8 is half an ulp of values in [1, 2)
    assert _one_pair(mod, "bf16", 0x3B80, 0x3F81, ONE["bf16"], ONE["bf16"])[1] == 0x3F82
    assert _one_pair(mod, "bf16", 0x3B80, 0x3F82, ONE["bf16"], ONE["bf16"])[1] == 0x3F82
    # overflow: 65504 + 16 is halfway to the next step and rounds to infinity; 65504 + 8 does not
    assert _one_pair(mod, "fp16", 0x4C00, 0x7BFF, ONE["fp16"], ONE["fp16"])[1] == INF["fp16"]  # 16
    assert _one_pair(mod, "fp16", 0x4800, 0x7BFF, ONE["fp16"], ONE["fp16"])[1] == 0x7BFF  # 8
    assert _one_pair(mod, "fp16", 0xCC00, 0xFBFF, ONE["fp16"], ONE["fp16"])[1] == 0xFC00
    # first output = a * 1 - b * 1: exact cancellation gives +0
    assert _one_pair(mod, "fp16", 0x3C01, 0x3C01, ONE["fp16"], ONE["fp16"])[0] == 0


def pin_relative_position(mod):
    fmt = "fp16"
    d, h = 32, 16
    q = _randn_bits((1, 1, d), fmt, 20)
    k = _randn_bits((1, 1, d), fmt, 21)
    inv = 10000.0 ** (-np.arange(h) * 2.0 / d)

    def table(p):
        th = np.concatenate([p * inv, p * inv])[None, :]
        return (_bits(torch.from_numpy(np.cos(th)).to(torch.float16)),
                _bits(torch.from_numpy(np.sin(th)).to(torch.float16)))

    def score(a, b):
        ca, sa = table(a)
        cb, sb = table(b)
        qa = _f64(mod.rope(q, ca, sa, fmt), fmt).ravel()
        kb = _f64(mod.rope(k, cb, sb, fmt), fmt).ravel()
        return float(qa @ kb)

    norm = float(np.linalg.norm(_f64(q, fmt)) * np.linalg.norm(_f64(k, fmt)))
    for a, b, t in ((7, 3, 50), (40, 45, 100), (100, 100, 17)):
        s0, s1 = score(a, b), score(a + t, b + t)
        assert abs(s0 - s1) <= 4e-3 * norm, f"score at ({a},{b}) vs ({a + t},{b + t}): {s0} vs {s1}"
    # and it does change with the distance
    assert abs(score(7, 3) - score(7, 30)) > 1e-2 * norm


def pin_pairs_only(mod):
    fmt = "bf16"
    d, h = 16, 8
    x = _randn_bits((1, 1, d), fmt, 22)
    c, s = _angle_tables(1, d, fmt, 23)
    base = mod.rope(x, c, s, fmt)
    for j in (0, 5, 8, 13):
        y = x.copy()
        y[0, 0, j] ^= 0x4000  # a large change of one input
        diff = np.nonzero(mod.rope(y, c, s, fmt) != base)[2].tolist()
        assert set(diff) <= {j, (j + h) % d}, f"changing input {j} changed outputs {diff}"
        assert diff, f"changing input {j} changed nothing"


ALL_PINS = [pin_identity, pin_quarter_turn, pin_half_turn, pin_complex_multiply, pin_operator_matrix,
            pin_bf16_exact_sums, pin_rounding_ties, pin_relative_position, pin_pairs_only]
