"""Rotary position embedding before the cache write (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module; it shares no code with the GPU library.

The decode step of the MiniCPM4 forward pass ("VoxCPM #395", the replacement
forward_step in section 4) applies ``apply_rotary_pos_emb(query, key, cos,
sin)`` to the new token's query and key just before the key and value rows
are written into the preallocated cache at position_id, and attends with the
rotated query. The page names that function without printing it; this module
takes the rotate-half form of the Llama-family code it comes from, element by
element over a head of D values (D even, h = D / 2):

    out[i] = x[i] * cos[i] - x[i + h] * sin[i]      for i <  h
    out[i] = x[i] * cos[i] + x[i - h] * sin[i]      for i >= h

with cos and sin given by the caller for the token's position (one row of D
values per batch row, in the same 16-bit format as x), so no frequency is
computed here. The result is the exact value of that expression over the
stored 16-bit inputs, rounded once to the nearest value of the format with
ties to even (overflow gives an infinity of the right sign); a zero result is
stored as +0. Inputs must be finite.

Everything is computed with exact rationals (``fractions.Fraction``) and the
rounding is a search in the sorted table of the format's finite values, so
the module is slow and meant for the small per-step tensors it is applied to
(batch x heads x D values).
"""
from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np

_TABLES: dict[str, tuple[list[float], list[int]]] = {}


def decode16(bits: int, fmt: str) -> float:
    """Value of one 16-bit pattern as a Python float (exact: both formats fit a double)."""
    bits = int(bits) & 0xFFFF
    sign = -1.0 if bits & 0x8000 else 1.0
    if fmt == "fp16":  # 1 sign, 5 exponent (bias 15), 10 fraction bits
        expo = (bits >> 10) & 0x1F
        frac = bits & 0x3FF
        if expo == 0x1F:
            return sign * float("inf") if frac == 0 else float("nan")
        if expo == 0:
            return sign * frac * 2.0 ** -24
        return sign * (1.0 + frac / 1024.0) * 2.0 ** (expo - 15)
    if fmt == "bf16":  # 1 sign, 8 exponent (bias 127), 7 fraction bits
        expo = (bits >> 7) & 0xFF
        frac = bits & 0x7F
        if expo == 0xFF:
            return sign * float("inf") if frac == 0 else float("nan")
        if expo == 0:
            return sign * frac * 2.0 ** -133
        return sign * (1.0 + frac / 128.0) * 2.0 ** (expo - 127)
    raise ValueError(f"unknown format {fmt}")


def _table(fmt: str) -> tuple[list[float], list[int]]:
    """Sorted non-negative finite values of the format and their bit patterns."""
    if fmt not in _TABLES:
        inf_bits = 0x7C00 if fmt == "fp16" else 0x7F80
        pairs = [(decode16(b, fmt), b) for b in range(0, inf_bits)]  # +0 up to the largest finite value
        _TABLES[fmt] = ([v for v, _ in pairs], [b for _, b in pairs])
    return _TABLES[fmt]


def round_to_format(value: Fraction, fmt: str) -> int:
    """Bit pattern of the format value nearest to ``value``, ties to the even pattern."""
    values, bits = _table(fmt)
    sign = 0x8000 if value < 0 else 0
    mag = -value if value < 0 else value
    if mag == 0:
        return 0
    top = Fraction(values[-1])
    top_ulp = top - Fraction(values[-2])
    # Past the largest finite value the next step would be one ulp further
    # (the infinity's place); halfway to it rounds to the even pattern, which
    # is the infinity since the largest finite pattern is odd.
    if mag >= top + top_ulp / 2:
        return sign | (0x7C00 if fmt == "fp16" else 0x7F80)
    j = bisect.bisect_left(values, mag)  # values[j - 1] < mag <= values[j]
    if j == len(values):  # above the largest value but less than halfway past it
        return sign | bits[-1]
    if values[j] == mag:
        return sign | bits[j]
    lo, hi = Fraction(values[j - 1]), Fraction(values[j])
    below, above = mag - lo, hi - mag
    if below < above:
        pick = bits[j - 1]
    elif above < below:
        pick = bits[j]
    else:
        pick = bits[j - 1] if bits[j - 1] % 2 == 0 else bits[j]
    return sign | pick


def rotate_half_exact(x: list[Fraction], cos: list[Fraction], sin: list[Fraction]) -> list[Fraction]:
    """The rotate-half rotary map of one head, in exact arithmetic."""
    d = len(x)
    h = d // 2
    out = []
    for i in range(d):
        if i < h:
            out.append(x[i] * cos[i] - x[i + h] * sin[i])
        else:
            out.append(x[i] * cos[i] + x[i - h] * sin[i])
    return out


def rope(x_bits: np.ndarray, cos_bits: np.ndarray, sin_bits: np.ndarray, fmt: str) -> np.ndarray:
    """Rotate every head of x.

    x_bits: uint16 patterns [B, H, D]; cos_bits, sin_bits: uint16 patterns
    [B, D] (row b is the table of batch row b's position). Returns the rotated
    heads as uint16 patterns [B, H, D].
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    cos_bits = np.asarray(cos_bits, dtype=np.uint16)
    sin_bits = np.asarray(sin_bits, dtype=np.uint16)
    if x_bits.ndim != 3:
        raise ValueError("x must be [B, H, D]")
    batch, heads, d = x_bits.shape
    if d % 2 or cos_bits.shape != (batch, d) or sin_bits.shape != (batch, d):
        raise ValueError("cos and sin must be [B, D] with D even")
    out = np.zeros_like(x_bits)
    for b in range(batch):
        c = [Fraction(decode16(v, fmt)) for v in cos_bits[b]]
        s = [Fraction(decode16(v, fmt)) for v in sin_bits[b]]
        for hd in range(heads):
            x = [Fraction(decode16(v, fmt)) for v in x_bits[b, hd]]
            y = rotate_half_exact(x, c, s)
            out[b, hd] = [round_to_format(v, fmt) for v in y]
    return out
