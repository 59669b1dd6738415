"""Pins for the CPU oracle: results obtained other than by the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages and the mathematics fix. They
are run against the real oracle by ``test_oracle_pins.py`` and against
deliberately broken copies of the oracle source by ``test_oracle_mutants.py``
(every such copy must fail at least one pin).

Pages (cited by title and section):
  [DECODE-FASTPATH] Cuda-Compute-OSS #343, "one-token decode fast path ...".
  [ACTIVE-PREFIX]   fish-speech #1310, "Optimize native AR decoding by
                    attending only to the active KV-cache prefix".
  [FORWARD-STEP]    VoxCPM #395, "MiniCPM4 MiniCPMAttention.forward_step
                    Attention Performance Fix".
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import workloads as W

SHAPE_GRID = [  # (n_head, n_kv_head, head_dim)
    (1, 1, 1), (1, 1, 128), (4, 1, 3), (4, 2, 8), (8, 2, 128), (32, 8, 8), (32, 8, 128), (6, 3, 5),
]
LEN_CHOICES = (1, 2, 3, 7, 16, 65)


def _shape(batch, hq, hkv, d, cap, dtype):
    return W.DecodeShape(batch, hq, hkv, d, cap, dtype)


def _f64(t: torch.Tensor) -> torch.Tensor:
    """torch's own 16-bit -> float64 conversion (independent of the oracle's decoders)."""
    return t.to(torch.float64)


def _sdpa_reference(q, k, v, lens, scale):
    """The pages' own call: SDPA on the active-prefix slice with enable_gqa
    ([FORWARD-STEP] section 4), in float64 on the CPU, one batch row at a time
    because rows may have different lengths."""
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    B, Hq, D = qd.shape
    out = torch.zeros((B, Hq, D), dtype=torch.float64)
    for b in range(B):
        n = max(0, min(int(lens[b]), kd.shape[2]))
        if n == 0:
            continue
        o = F.scaled_dot_product_attention(qd[b:b + 1, :, None, :], kd[b:b + 1, :, :n, :].contiguous(),
                                           vd[b:b + 1, :, :n, :].contiguous(), scale=scale, enable_gqa=True)
        out[b] = o[0, :, 0, :]
    return out.numpy()


def _close(a, b, rel=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite oracle output"
    denom = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rel * denom, f"{what}: max abs diff {err:.3e} > {rel:.1e} * {denom:.3e}"


# ---------------------------------------------------------------------------
# 16-bit decoders: exhaustive over all bit patterns.


def pin_f16_decoder_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = o.decode_bits(bits, "fp16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "fp16 decoder: NaN patterns differ"
    assert np.array_equal(got[~nan], want[~nan]), "fp16 decoder: value mismatch"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "fp16 decoder: sign of zero"


def pin_bf16_decoder_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = o.decode_bits(bits, "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "bf16 decoder: NaN patterns differ"
    assert np.array_equal(got[~nan], want[~nan]), "bf16 decoder: value mismatch"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "bf16 decoder: sign of zero"


# ---------------------------------------------------------------------------
# Whole oracle against an independent library implementation of attention.


def pin_matches_library_sdpa_gqa(o):
    """Active-prefix GQA attention equals torch's float64 SDPA with enable_gqa on
    the sliced cache ([FORWARD-STEP] section 4; [ACTIVE-PREFIX] section 2)."""
    case = 0
    for dtype in ("fp16", "bf16"):
        for hq, hkv, d in SHAPE_GRID:
            batch = 1 + case % 3
            cap = 80
            g = torch.Generator().manual_seed(1000 + case)
            lens = [LEN_CHOICES[int(i)] for i in torch.randint(0, len(LEN_CHOICES), (batch,), generator=g)]
            x = W.decode_inputs(_shape(batch, hq, hkv, d, cap, dtype), lens, seed=2000 + case, tail="nan")
            scale = 1.0 / math.sqrt(d)
            got = o.decode(x["q"], x["k_cache"], x["v_cache"], lens, scale)
            want = _sdpa_reference(x["q"], x["k_cache"], x["v_cache"], lens, scale)
            _close(got, want, 1e-12, f"sdpa {dtype} hq={hq} hkv={hkv} d={d} lens={lens}")
            case += 1


def pin_equals_masked_full_capacity(o):
    """Slicing to the active prefix equals attention over the whole cache with a
    boolean mask admitting slots 0..position_id only (the removed baseline of
    [FORWARD-STEP] section 2.1; [ACTIVE-PREFIX] section 1)."""
    for dtype, (hq, hkv, d), cap, pos in (("fp16", (8, 2, 16), 64, 20), ("bf16", (32, 8, 128), 96, 0),
                                          ("fp16", (4, 4, 8), 33, 32)):
        x = W.decode_inputs(_shape(1, hq, hkv, d, cap, dtype), [pos + 1], seed=77 + pos, tail="random")
        scale = 1.0 / math.sqrt(d)
        mask = (torch.arange(cap) <= pos)[None, None, None, :]
        want = F.scaled_dot_product_attention(_f64(x["q"])[:, :, None, :], _f64(x["k_cache"]),
                                              _f64(x["v_cache"]), attn_mask=mask, scale=scale,
                                              enable_gqa=True)[:, :, 0, :].numpy()
        got = o.decode(x["q"], x["k_cache"], x["v_cache"], [pos + 1], scale)
        _close(got, want, 1e-12, f"masked full capacity pos={pos}")


def pin_large_scores_stable(o):
    """Scores in the thousands: the max-subtracted softmax stays finite and
    matches the library ([DECODE-FASTPATH], "Correctness risks")."""
    for dtype in ("fp16", "bf16"):
        x = W.decode_inputs(_shape(2, 4, 2, 32, 40, dtype), [40, 17], seed=5, tail="random")
        k = (x["k_cache"].to(torch.float32) * 64).to(x["k_cache"].dtype)  # exact power-of-two scaling
        q = (x["q"].to(torch.float32) * 16).to(x["q"].dtype)
        got = o.decode(q, k, x["v_cache"], [40, 17], 1.0)
        want = _sdpa_reference(q, k, x["v_cache"], [40, 17], 1.0)
        _close(got, want, 1e-10, f"large scores {dtype}")


# ---------------------------------------------------------------------------
# Grouped-query head sharing.


def pin_gqa_equals_repeat_interleave_mha(o):
    """GQA equals plain multi-head attention on K/V expanded with
    repeat_interleave ([ACTIVE-PREFIX] section 1, the expansion the fix keeps
    out of the hot path)."""
    for hq, hkv in ((4, 2), (32, 8), (6, 3), (8, 1)):
        x = W.decode_inputs(_shape(2, hq, hkv, 16, 24, "fp16"), [24, 9], seed=hq * 10 + hkv, tail="nan")
        rep = hq // hkv
        k_mha = x["k_cache"].repeat_interleave(rep, dim=1)
        v_mha = x["v_cache"].repeat_interleave(rep, dim=1)
        got = o.decode(x["q"], x["k_cache"], x["v_cache"], [24, 9], 0.25)
        want = o.decode(x["q"], k_mha, v_mha, [24, 9], 0.25)
        _close(got, want, 1e-15, f"gqa vs mha {hq}/{hkv}")


def pin_gqa_head_map_closed_form(o):
    """With every value row of KV head g equal to the constant g + 1, query head
    h must return (h // G) + 1 everywhere: consecutive query heads share a KV
    head (repeat_interleave order), not h mod n_kv_head."""
    hq, hkv, d, cap = 12, 3, 8, 10
    x = W.decode_inputs(_shape(2, hq, hkv, d, cap, "bf16"), [10, 4], seed=3, tail="nan")
    v = x["v_cache"].clone()
    for g in range(hkv):
        v[:, g, :, :] = float(g + 1)
    got = o.decode(x["q"], x["k_cache"], v, [10, 4], 0.3)
    group = hq // hkv
    want = np.zeros_like(got)
    for h in range(hq):
        want[:, h, :] = h // group + 1
    _close(got, want, 1e-13, "gqa head map")


# ---------------------------------------------------------------------------
# Closed forms and special cases.


def pin_single_slot_returns_v0(o):
    """kv_len = 1 (position_id 0): softmax over one entry is the identity, so
    the output is v[0] exactly ([FORWARD-STEP] section 3)."""
    for dtype in ("fp16", "bf16"):
        x = W.decode_inputs(_shape(3, 8, 2, 128, 16, dtype), [1, 1, 1], seed=11, tail="nan")
        got = o.decode(x["q"], x["k_cache"], x["v_cache"], [1, 1, 1], 0.088388)
        want = _f64(x["v_cache"][:, :, 0, :]).repeat_interleave(4, dim=1).numpy()
        assert np.array_equal(got, want), f"kv_len=1 must return v[0] exactly ({dtype})"


def pin_uniform_weights_mean(o):
    """Equal scores (scale 0, zero query, or identical keys) give the plain
    mean of the active value rows."""
    shp = _shape(2, 4, 2, 16, 30, "fp16")
    lens = [30, 7]
    x = W.decode_inputs(shp, lens, seed=21, tail="nan")
    vd = _f64(x["v_cache"])
    want = np.zeros((2, 4, 16))
    for b, n in enumerate(lens):
        m = vd[b, :, :n, :].mean(dim=1).numpy()  # [Hkv, D]
        want[b] = np.repeat(m, 2, axis=0)
    got0 = o.decode(x["q"], x["k_cache"], x["v_cache"], lens, 0.0)
    _close(got0, want, 1e-13, "scale 0")
    gotq = o.decode(torch.zeros_like(x["q"]), x["k_cache"], x["v_cache"], lens, 0.7)
    _close(gotq, want, 1e-13, "zero query")
    k_same = x["k_cache"].clone()
    k_same[:, :, :, :] = x["k_cache"][:, :, :1, :]
    gotk = o.decode(x["q"], k_same, x["v_cache"], lens, 0.7)
    _close(gotk, want, 1e-13, "identical keys")


def pin_two_keys_closed_form(o):
    """Two slots: out = s * v0 + (1 - s) * v1 with s = 1 / (1 + exp(x1 - x0)).
    Small-integer inputs make the dot products exact."""
    g = torch.Generator().manual_seed(8)
    d = 8
    q = torch.randint(-3, 4, (1, 2, d), generator=g).to(torch.float16)
    k = torch.randint(-3, 4, (1, 1, 2, d), generator=g).to(torch.float16)
    v = torch.randn((1, 1, 2, d), generator=g).to(torch.float16)
    scale = 0.37
    got = o.decode(q, k, v, [2], scale)
    qi, ki, vd = q.to(torch.int64), k.to(torch.int64), _f64(v)
    for h in range(2):
        x0 = scale * int((qi[0, h] * ki[0, 0, 0]).sum())
        x1 = scale * int((qi[0, h] * ki[0, 0, 1]).sum())
        s = 1.0 / (1.0 + math.exp(x1 - x0))
        want = s * vd[0, 0, 0].numpy() + (1.0 - s) * vd[0, 0, 1].numpy()
        _close(got[0, h], want, 1e-14, f"two keys head {h}")


# ---------------------------------------------------------------------------
# Invariants of softmax attention.


def _int_inputs(seed, batch, hq, hkv, d, cap, lo=-4, hi=5, dtype=torch.float16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(lo, hi, (batch, hq, d), generator=g).to(dtype)
    k = torch.randint(lo, hi, (batch, hkv, cap, d), generator=g).to(dtype)
    v = torch.randint(lo, hi, (batch, hkv, cap, d), generator=g).to(dtype)
    return q, k, v


def pin_key_shift_invariance(o):
    """Adding one vector u to every key shifts all scores of a head by q.u and
    leaves the output unchanged (inputs chosen so K + u is exact)."""
    q, k, v = _int_inputs(31, 2, 4, 2, 8, 12)
    u = torch.randint(-3, 4, (8,), generator=torch.Generator().manual_seed(32)).to(torch.float16)
    lens = [12, 5]
    a = o.decode(q, k, v, lens, 0.11)
    b = o.decode(q, k + u, v, lens, 0.11)
    _close(a, b, 1e-12, "key shift")


def pin_permutation_invariance(o):
    """Reordering the (key, value) pairs of the active prefix leaves the output
    unchanged; the tail is untouched."""
    x = W.decode_inputs(_shape(1, 8, 2, 16, 20, "bf16"), [13], seed=41, tail="nan")
    perm = torch.randperm(13, generator=torch.Generator().manual_seed(42))
    k, v = x["k_cache"].clone(), x["v_cache"].clone()
    k[:, :, :13] = x["k_cache"][:, :, perm]
    v[:, :, :13] = x["v_cache"][:, :, perm]
    a = o.decode(x["q"], x["k_cache"], x["v_cache"], [13], 0.25)
    b = o.decode(x["q"], k, v, [13], 0.25)
    _close(a, b, 1e-13, "permutation")


def pin_convex_combination(o):
    """Each output is a convex combination of the active value rows, so it lies
    inside their per-dimension range."""
    lens = [50, 3]
    x = W.decode_inputs(_shape(2, 8, 4, 32, 64, "fp16"), lens, seed=51, tail="nan")
    got = o.decode(x["q"], x["k_cache"], x["v_cache"], lens, 0.17)
    vd = _f64(x["v_cache"])
    for b, n in enumerate(lens):
        lo = vd[b, :, :n].min(dim=1).values.repeat_interleave(2, dim=0).numpy()
        hi = vd[b, :, :n].max(dim=1).values.repeat_interleave(2, dim=0).numpy()
        assert np.all(got[b] >= lo - 1e-12) and np.all(got[b] <= hi + 1e-12), "outside the value hull"


def pin_linear_in_values(o):
    """For fixed q and K the output is linear in V (exactly representable
    combination a*V1 + b*V2)."""
    q, k, v1 = _int_inputs(61, 1, 4, 2, 8, 10)
    _, _, v2 = _int_inputs(62, 1, 4, 2, 8, 10)
    v3 = (3 * v1.to(torch.float32) - 2 * v2.to(torch.float32)).to(torch.float16)
    a = o.decode(q, k, v1, [10], 0.2)
    b = o.decode(q, k, v2, [10], 0.2)
    c = o.decode(q, k, v3, [10], 0.2)
    _close(c, 3 * a - 2 * b, 1e-12, "linearity")


def pin_scale_is_key_scaling(o):
    """Doubling the scale equals doubling every key (an exact scaling)."""
    x = W.decode_inputs(_shape(2, 4, 2, 16, 25, "fp16"), [25, 11], seed=71, tail="nan")
    k2 = (x["k_cache"].to(torch.float32) * 2).to(torch.float16)
    a = o.decode(x["q"], x["k_cache"], x["v_cache"], [25, 11], 0.5)
    b = o.decode(x["q"], k2, x["v_cache"], [25, 11], 0.25)
    _close(a, b, 1e-13, "scale vs key scaling")


# ---------------------------------------------------------------------------
# Active-prefix edges.


def pin_empty_and_clamped_lengths(o):
    """kv_len 0 or negative gives zeros (empty sum); kv_len beyond the capacity
    is clamped to the capacity."""
    x = W.decode_inputs(_shape(3, 4, 2, 8, 16, "bf16"), [16, 16, 16], seed=81, tail="random")
    got = o.decode(x["q"], x["k_cache"], x["v_cache"], [0, -5, 1000], 0.3)
    assert np.array_equal(got[0], np.zeros_like(got[0])), "kv_len 0 must give zeros"
    assert np.array_equal(got[1], np.zeros_like(got[1])), "negative kv_len must give zeros"
    full = o.decode(x["q"], x["k_cache"], x["v_cache"], [16, 16, 16], 0.3)
    assert np.array_equal(got[2], full[2]), "kv_len beyond capacity must clamp"


def pin_tail_never_read(o):
    """The same inputs with a NaN tail and with a random tail give identical
    outputs: no slot at or beyond kv_len is read ([ACTIVE-PREFIX] section 2)."""
    shp = _shape(2, 8, 2, 16, 40, "fp16")
    lens = [9, 31]
    a = W.decode_inputs(shp, lens, seed=91, tail="random")
    b = {k: t.clone() for k, t in a.items()}
    for i, n in enumerate(lens):
        b["k_cache"][i, :, n:] = float("nan")
        b["v_cache"][i, :, n:] = float("nan")
    ra = o.decode(a["q"], a["k_cache"], a["v_cache"], lens, 0.25)
    rb = o.decode(b["q"], b["k_cache"], b["v_cache"], lens, 0.25)
    assert np.all(np.isfinite(rb)) and np.array_equal(ra, rb), "tail slots influenced the output"


def pin_batch_rows_independent(o):
    """A ragged batch equals each batch row computed on its own."""
    lens = [5, 40, 1, 23]
    x = W.decode_inputs(_shape(4, 8, 4, 16, 40, "bf16"), lens, seed=101, tail="nan")
    got = o.decode(x["q"], x["k_cache"], x["v_cache"], lens, 0.2)
    for b, n in enumerate(lens):
        one = o.decode(x["q"][b:b + 1], x["k_cache"][b:b + 1], x["v_cache"][b:b + 1], [n], 0.2)
        assert np.array_equal(got[b], one[0]), f"row {b} depends on other rows"


# ---------------------------------------------------------------------------
# In-place cache append.


def pin_kv_append_matches_index_assign(o):
    """Writing row pos[b] equals torch index assignment of the same rows
    ([FORWARD-STEP] section 4, cache write at position_id); rows with pos
    outside [0, capacity) write nothing."""
    B, Hkv, S, D = 4, 3, 10, 8
    x = W.decode_inputs(_shape(B, 6, Hkv, D, S, "fp16"), [S] * B, seed=111, tail="random")
    kn, vn = W.append_inputs(B, Hkv, D, "fp16", seed=112)
    pos = [0, 9, -1, 10]
    kc, vc = o.kv_append(kn, vn, x["k_cache"], x["v_cache"], pos)
    k_ref, v_ref = x["k_cache"].clone(), x["v_cache"].clone()
    for b, p in enumerate(pos):
        if 0 <= p < S:
            k_ref[b, :, p, :] = kn[b]
            v_ref[b, :, p, :] = vn[b]
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kc, bits(k_ref)), "kv_append K mismatch"
    assert np.array_equal(vc, bits(v_ref)), "kv_append V mismatch"


def pin_append_then_decode_is_forward_step(o):
    """One decode step as the pages run it: append at position_id, then attend
    over slots 0..position_id; equals the library SDPA on that slice
    ([FORWARD-STEP] section 4)."""
    B, Hq, Hkv, D, S = 2, 8, 2, 16, 32
    pos = 13
    x = W.decode_inputs(_shape(B, Hq, Hkv, D, S, "bf16"), [pos] * B, seed=121, tail="zero")
    kn, vn = W.append_inputs(B, Hkv, D, "bf16", seed=122)
    kc, vc = o.kv_append(kn, vn, x["k_cache"], x["v_cache"], [pos] * B)
    kc_t = torch.from_numpy(kc.view(np.int16)).view(torch.bfloat16)
    vc_t = torch.from_numpy(vc.view(np.int16)).view(torch.bfloat16)
    got = o.decode(x["q"], kc_t, vc_t, [pos + 1] * B, 0.25)
    want = _sdpa_reference(x["q"], kc_t, vc_t, [pos + 1] * B, 0.25)
    _close(got, want, 1e-12, "append then decode")


# ---------------------------------------------------------------------------
# Prefill: T query tokens per row at positions start[b] + t, causal.


def _prefill_inputs(B, Hq, Hkv, D, S, T, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    dt = W.TORCH_DTYPES[dtype]
    q = torch.randn((B, Hq, T, D), generator=g).to(dt)
    k = torch.randn((B, Hkv, S, D), generator=g).to(dt)
    v = torch.randn((B, Hkv, S, D), generator=g).to(dt)
    return q, k, v


def pin_prefill_matches_library_causal_sdpa(o):
    """Prompt prefill from slot 0 is SDPA with is_causal=True over the T prompt
    slots ([FORWARD-STEP] section 5: the batch prefill path keeps is_causal;
    [ACTIVE-PREFIX] section 2: kv_len = T after prefill), float64 on the CPU."""
    for (B, Hq, Hkv, D, T, dtype) in ((1, 4, 1, 16, 9, "fp16"), (2, 8, 2, 32, 17, "bf16"), (1, 32, 8, 128, 33, "fp16")):
        S = T + 5  # slots past the prompt hold values that must not be seen
        q, k, v = _prefill_inputs(B, Hq, Hkv, D, S, T, dtype, 600 + T)
        k[:, :, T:] = float("nan")
        v[:, :, T:] = float("nan")
        scale = 1.0 / math.sqrt(D)
        got = o.prefill(q, k, v, [0] * B, scale)
        want = F.scaled_dot_product_attention(_f64(q), _f64(k[:, :, :T]).contiguous(), _f64(v[:, :, :T]).contiguous(),
                                              is_causal=True, scale=scale, enable_gqa=True).numpy()
        _close(got, want, 1e-12, f"prefill vs causal SDPA {B}x{Hq}/{Hkv}x{T}x{D}")


def pin_prefill_continued_prompt_mask(o):
    """A prompt continued at start > 0: token t sees slots 0 .. start + t, the
    boolean mask j <= start + t over the first start + T slots (SDPA with an
    explicit mask; different rows, different starts)."""
    B, Hq, Hkv, D, S, T = 3, 8, 2, 32, 64, 7
    q, k, v = _prefill_inputs(B, Hq, Hkv, D, S, T, "bf16", 610)
    starts = [0, 10, 57]
    scale = 0.17
    got = o.prefill(q, k, v, starts, scale)
    for b, st in enumerate(starts):
        n = st + T
        mask = torch.arange(n)[None, :] <= (st + torch.arange(T))[:, None]
        want = F.scaled_dot_product_attention(_f64(q[b:b + 1]), _f64(k[b:b + 1, :, :n]).contiguous(),
                                              _f64(v[b:b + 1, :, :n]).contiguous(), attn_mask=mask, scale=scale,
                                              enable_gqa=True).numpy()
        _close(got[b:b + 1], want, 1e-12, f"continued prompt start={st}")


def pin_prefill_rows_are_decode_calls(o):
    """Each prefill token is a single-token decode over kv_len = start + t + 1
    (and the slots past a clamped position are the whole cache)."""
    B, Hq, Hkv, D, S, T = 2, 6, 3, 8, 20, 6
    q, k, v = _prefill_inputs(B, Hq, Hkv, D, S, T, "fp16", 620)
    starts = [3, 17]  # the second row runs past the cache: clamped to S slots
    got = o.prefill(q, k, v, starts, 0.3)
    for t in range(T):
        lens = [min(S, st + t + 1) for st in starts]
        want = _sdpa_reference(q[:, :, t, :], k, v, lens, 0.3)
        _close(got[:, :, t, :], want, 1e-12, f"prefill token {t}")


def pin_prefill_append_matches_slice_assign(o):
    """The prompt's rows land at slots start .. start + T - 1, bit for bit;
    rows outside the cache are dropped; nothing else changes."""
    B, Hkv, D, S, T = 3, 2, 8, 16, 5
    g = torch.Generator().manual_seed(630)
    kc = torch.randn((B, Hkv, S, D), generator=g).to(torch.float16)
    vc = torch.randn((B, Hkv, S, D), generator=g).to(torch.float16)
    kn = torch.randn((B, Hkv, T, D), generator=g).to(torch.float16)
    vn = torch.randn((B, Hkv, T, D), generator=g).to(torch.float16)
    starts = [0, 9, 13]
    got_k, got_v = o.prefill_append(kn, vn, kc, vc, starts)
    want_k, want_v = kc.clone(), vc.clone()
    for b, st in enumerate(starts):
        m = min(T, S - st)
        want_k[b, :, st:st + m] = kn[b, :, :m]
        want_v[b, :, st:st + m] = vn[b, :, :m]
    to_bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_k, to_bits(want_k)) and np.array_equal(got_v, to_bits(want_v)), "prefill append"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
