"""GPU parity on seeded random shapes: decode calls, decode steps and prompt
prefill (append + causal attention) against the fp64 oracle, through the C
ABI.

Each case draws batch, KV heads, group size (1..8), capacity, per-row live
lengths (including 0, 1 and the full capacity), dtype, scale (including 0 and
negative values) and a split count (heuristic or forced), so combinations the
hand-written cases do not name are still covered. Cache tails are NaN: a read
past a row's live prefix makes the output non-finite. The definition is the
one of [DECODE-FASTPATH] "Proposed implementation" over the active prefix
([ACTIVE-PREFIX] section 2) with query head h reading KV head h / G
([ACTIVE-PREFIX] section 1).
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_parity

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def ada():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import autoregressive_decode_attention_amd as m

    return m


@pytest.fixture(scope="module")
def ora():
    return oracle.load()


def draw_case(rng: random.Random):
    B = rng.choice([1, 1, 2, 3, 4, 6])
    Hkv = rng.choice([1, 2, 3, 4, 8])
    G = rng.randint(1, 8)
    S = rng.choice([1, 7, 64, 65, 300, 1000, 2049, 3000])
    lens = []
    for _ in range(B):
        kind = rng.random()
        lens.append(0 if kind < 0.1 else 1 if kind < 0.2 else S if kind < 0.35 else rng.randint(1, S))
    dtype = rng.choice(["fp16", "bf16"])
    scale = rng.choice([float(np.float32(1 / math.sqrt(128)))] * 3 + [0.5, -0.3, 0.0])
    splits = rng.choice([0, 0, 1, 2, 3, 7, 16, 40])
    return B, Hkv, G, S, lens, dtype, scale, splits


@pytest.mark.parametrize("seed", range(40))
def test_random_decode(ada, ora, seed):
    rng = random.Random(7100 + seed)
    B, Hkv, G, S, lens, dtype, scale, splits = draw_case(rng)
    Hq = Hkv * G
    say(f"case random decode {seed}: B={B} Hq={Hq} Hkv={Hkv} S={S} {dtype} lens={lens} scale={scale} splits={splits}")
    x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, 128, S, dtype), lens, 7200 + seed, tail="nan")
    d = {k: v.cuda() for k, v in x.items()}
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = ada.decode_attn_gqa_ex(d["q"], d["k_cache"], d["v_cache"], lens_t, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], lens, scale)
    assert_parity(out, want, dtype, f"random decode {seed}")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[b]) == 0, "an empty row must give zeros"


@pytest.mark.parametrize("seed", range(12))
def test_random_decode_step(ada, ora, seed):
    """Append at device positions then attend over pos + 1 slots; the cache
    rows written must be the new rows bit for bit."""
    rng = random.Random(7300 + seed)
    B, Hkv, G, S, _, dtype, scale, splits = draw_case(rng)
    S = max(S, 2)
    Hq = Hkv * G
    pos = [rng.randint(0, S - 1) for _ in range(B)]
    say(f"case random decode step {seed}: B={B} Hq={Hq} Hkv={Hkv} S={S} {dtype} pos={pos} scale={scale} splits={splits}")
    x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, 128, S, dtype), pos, 7400 + seed, tail="nan")
    kn, vn = W.append_inputs(B, Hkv, 128, dtype, 7500 + seed)
    d = {k: v.cuda() for k, v in x.items()}
    pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = ada.decode_step(d["q"], kn.cuda(), vn.cuda(), d["k_cache"], d["v_cache"], pos_t, scale=scale,
                          max_pos=max(pos), num_splits=splits)
    torch.cuda.synchronize()
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    for b, p in enumerate(pos):
        kc[b, :, p] = kn[b]
        vc[b, :, p] = vn[b]
    assert torch.equal(d["k_cache"].cpu().view(torch.int16), kc.view(torch.int16))
    assert torch.equal(d["v_cache"].cpu().view(torch.int16), vc.view(torch.int16))
    want = ora.decode(x["q"], kc, vc, [p + 1 for p in pos], scale)
    assert_parity(out, want, dtype, f"random decode step {seed}")


@pytest.mark.parametrize("seed", range(16))
def test_random_prefill(ada, ora, seed):
    """Prompt append then causal prefill attention from random starts
    (including 0, continued prompts and prompts running past the cache):
    appended rows bit for bit, outputs within the decode's tolerances. Slots
    no token may see hold NaN. Prompt lengths reach past one 64-row block so
    both workgroup sizes and ragged row tiles occur."""
    random_prefill_case(ada, ora, seed)


# Draws of the case above (beyond the committed seeds) on which softmax
# weights rounded once to bf16 in the value product would miss the bf16
# max-abs: a CPU model of that arithmetic (exact weights rounded to nearest
# even, the row sums of the rounded weights, output rounded) puts their
# largest error at 1.5e-2 .. 1.6e-2 of the 1.6e-2 bar. The kernel carries
# each weight as a pair of 16-bit values, so these must pass with margin.
WEIGHT_ROUNDING_SEEDS = (26, 250, 485, 676, 913, 918, 922)


@pytest.mark.parametrize("seed", WEIGHT_ROUNDING_SEEDS)
def test_random_prefill_weight_rounding(ada, ora, seed):
    random_prefill_case(ada, ora, seed)


def random_prefill_case(ada, ora, seed):
    rng = random.Random(7600 + seed)
    B = rng.choice([1, 2, 3, 4])
    Hkv = rng.choice([1, 2, 4, 8])
    G = rng.randint(1, 8)
    Hq = Hkv * G
    S = rng.choice([16, 100, 300, 700, 1500])
    T = rng.randint(1, min(S, 400))
    dtype = rng.choice(["fp16", "bf16"])
    scale = rng.choice([float(np.float32(1 / math.sqrt(128)))] * 3 + [0.5, -0.3, 0.0])
    starts = [rng.choice([0, 0, rng.randint(0, S - 1), S - T // 2]) for _ in range(B)]
    say(f"case random prefill {seed}: B={B} Hq={Hq} Hkv={Hkv} S={S} T={T} {dtype} starts={starts} scale={scale}")
    g = torch.Generator().manual_seed(7700 + seed)
    dt = W.TORCH_DTYPES[dtype]
    q = torch.randn((B, Hq, T, 128), generator=g).to(dt)
    kc = torch.randn((B, Hkv, S, 128), generator=g).to(dt)
    vc = torch.randn((B, Hkv, S, 128), generator=g).to(dt)
    kn = torch.randn((B, Hkv, T, 128), generator=g).to(dt)
    vn = torch.randn((B, Hkv, T, 128), generator=g).to(dt)
    for b, st in enumerate(starts):  # slots past the prompt's end are never visible
        end = max(0, min(S, st + T))
        kc[b, :, end:] = float("nan")
        vc[b, :, end:] = float("nan")
    d_kc, d_vc = kc.cuda(), vc.cuda()
    st_t = torch.tensor(starts, dtype=torch.int32, device="cuda")
    ada.prefill_append(kn.cuda(), vn.cuda(), d_kc, d_vc, st_t)
    out = ada.prefill_attn_gqa(q.cuda(), d_kc, d_vc, st_t, scale=scale)
    torch.cuda.synchronize()
    want_kc, want_vc = kc.clone(), vc.clone()
    for b, st in enumerate(starts):
        for t in range(T):
            if 0 <= st + t < S:
                want_kc[b, :, st + t] = kn[b, :, t]
                want_vc[b, :, st + t] = vn[b, :, t]
    assert torch.equal(d_kc.cpu().view(torch.int16), want_kc.view(torch.int16))
    assert torch.equal(d_vc.cpu().view(torch.int16), want_vc.view(torch.int16))
    want = ora.prefill(q, want_kc, want_vc, starts, scale)
    assert_parity(out, want, dtype, f"random prefill {seed}")


@pytest.mark.parametrize("seed", range(12))
def test_random_rope_step(ada, ora, seed):
    """Rotary decode steps (ada_decode_step_rope) on random shapes and
    per-row positions -- including 0, the last slot, negative and past the
    cache -- with heuristic (balanced for several rows) or forced splits:
    rotated key rows bit for bit, outputs within tolerance of the oracle
    (oracle/rope.py composed with the append and decode oracles)."""
    from test_gpu_rope import rope_step_case

    rng = random.Random(7800 + seed)
    B = rng.choice([1, 2, 3, 4, 6])
    Hkv = rng.choice([1, 2, 4, 8])
    G = rng.randint(1, 8)
    S = rng.choice([64, 65, 300, 1000, 2049])
    pos = [rng.choice([0, S - 1, rng.randint(0, S - 1), rng.randint(0, S - 1), -1, S]) for _ in range(B)]
    dtype = rng.choice(["fp16", "bf16"])
    splits = rng.choice([0, 0, 1, 3, 16])
    rope_step_case(ada, ora, B, Hkv * G, Hkv, S, dtype, pos, 7900 + 10 * seed, splits)
