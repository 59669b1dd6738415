"""GPU parity of the prompt prefill: ada_prefill_append (bit-exact) and
ada_prefill_attn_gqa (causal, matrix cores) against the oracle, through the C
ABI.

Prefill is read from [ACTIVE-PREFIX] (fish-speech #1310, "Optimize native AR
decoding by attending only to the active KV-cache prefix", section 2:
kv_len = T after the prompt) and [FORWARD-STEP] (VoxCPM #395, "MiniCPM4
MiniCPMAttention.forward_step Attention Performance Fix", section 5: the
batch prefill path keeps is_causal=True): token t at position start + t sees
cache slots 0 .. start + t. Tolerances: those of the decode (max-abs 4e-3 /
relative Frobenius 1e-3 for fp16, 1.6e-2 / 4e-3 for bf16, over the whole
output of a call); cache slots no token may see hold NaN.
"""
import math

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


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def prefill_inputs(B, Hq, Hkv, T, S, dtype, starts, seed):
    """q [B, Hq, T, D]; caches with finite slots 0 .. start + T - 1 and NaN beyond."""
    g = torch.Generator().manual_seed(seed)
    dt = W.TORCH_DTYPES[dtype]
    q = torch.randn((B, Hq, T, 128), generator=g).to(dt)
    k = torch.randn((B, Hkv, S, 128), generator=g).to(dt)
    v = torch.randn((B, Hkv, S, 128), generator=g).to(dt)
    for b, st in enumerate(starts):
        n = max(0, min(S, st + T))
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    return q, k, v


def check_prefill(out, want, dtype, what):
    return assert_parity(out, want, dtype, what)


def run_prefill(ada, ora, B, Hq, Hkv, T, S, dtype, starts, seed, what=""):
    say(f"case prefill {what}: B={B} Hq={Hq} Hkv={Hkv} T={T} S={S} {dtype} starts={starts} seed={seed}")
    q, k, v = prefill_inputs(B, Hq, Hkv, T, S, dtype, starts, seed)
    scale = 1.0 / math.sqrt(128)
    st = None if all(s == 0 for s in starts) else torch.tensor(starts, dtype=torch.int32, device="cuda")
    out = ada.prefill_attn_gqa(q.cuda(), k.cuda(), v.cuda(), st, scale=scale)
    torch.cuda.synchronize()
    want = ora.prefill(q, k, v, starts, scale)
    check_prefill(out, want, dtype, what)
    return q, k, v, out


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_prefill_append_bit_exact(ada, ora, dtype):
    B, Hkv, T, S = 3, 8, 70, 128
    starts = [0, 20, 100]  # the last runs past the cache: its late rows are dropped
    say(f"case prefill_append {dtype} starts={starts}")
    g = torch.Generator().manual_seed(800)
    dt = W.TORCH_DTYPES[dtype]
    kc = torch.randn((B, Hkv, S, 128), generator=g).to(dt)
    vc = torch.randn((B, Hkv, S, 128), generator=g).to(dt)
    kn = torch.randn((B, Hkv, T, 128), generator=g).to(dt)
    vn = torch.randn((B, Hkv, T, 128), generator=g).to(dt)
    kd, vd = kc.cuda(), vc.cuda()
    ada.prefill_append(kn.cuda(), vn.cuda(), kd, vd, starts)
    torch.cuda.synchronize()
    want_k, want_v = ora.prefill_append(kn, vn, kc, vc, starts)
    assert np.array_equal(bits(kd), want_k) and np.array_equal(bits(vd), want_v)
    kd2, vd2 = kc.cuda(), vc.cuda()
    ada.prefill_append(kn.cuda(), vn.cuda(), kd2, vd2)  # start None: slot 0
    torch.cuda.synchronize()
    want_k0, want_v0 = ora.prefill_append(kn, vn, kc, vc, [0] * B)
    assert np.array_equal(bits(kd2), want_k0) and np.array_equal(bits(vd2), want_v0)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_prefill_s2pro_prompt(ada, ora, dtype):
    """The S2-Pro prompt: 234 tokens, 32/8 heads, from slot 0 of a 32768-slot cache."""
    run_prefill(ada, ora, 1, 32, 8, 234, 32768, dtype, [0], W.seed_for(2, 50_000), "s2pro prompt")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 8])
def test_prefill_group_sizes(ada, ora, dtype, group):
    """Every lane layout of the row tiles: G heads interleaved per token, ragged
    tails of the 64-row tiles, continued prompts (start > 0)."""
    Hkv = 2
    run_prefill(ada, ora, 2, Hkv * group, Hkv, 77, 512, dtype, [0, 131], 810 + group, f"G={group}")


def test_prefill_edges(ada, ora):
    """One token (a decode), a prompt ending at the last slot, starts past the
    cache (clamped to the capacity), tiny caches, T not a multiple of 16."""
    run_prefill(ada, ora, 2, 8, 2, 1, 300, "fp16", [0, 299], 830, "T=1")
    run_prefill(ada, ora, 1, 32, 8, 64, 64, "bf16", [0], 831, "fills the cache")
    run_prefill(ada, ora, 2, 16, 4, 40, 100, "fp16", [70, 100], 832, "past the cache")
    run_prefill(ada, ora, 3, 4, 4, 13, 16, "bf16", [0, 1, 3], 833, "tiny cache")


def test_prefill_long_prompt(ada, ora):
    """A 1024-token prompt (16 row tiles per head group, 16 key tiles for the last)."""
    run_prefill(ada, ora, 1, 32, 8, 1024, 2048, "bf16", [0], 840, "long prompt")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_prefill_two_row_blocks(ada, ora, dtype):
    """Launches large enough for 128-row workgroups (two 16-row blocks per
    wavefront, every K and V operand read serving both): the rule picks them
    on this device, and the results match the oracle with ragged starts and
    with a last row tile whose upper two wavefronts hold no row."""
    cases = [(16, 32, 8, 256, 600, [0, 7, 100, 333, 0, 1, 64, 200, 5, 9, 300, 17, 0, 250, 128, 40]),  # G = 4
             (32, 64, 8, 72, 200, [3 * i for i in range(32)])]  # G = 8: 576 rows, last tile 64 of 128
    for k, (B, Hq, Hkv, T, S, starts) in enumerate(cases):
        assert ada.prefill_rows_per_workgroup(B, Hq, Hkv, T) == 128, "this case must take the two-block path"
        run_prefill(ada, ora, B, Hq, Hkv, T, S, dtype, starts, 880 + k, f"two row blocks {k}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_prefill_full_size_sampled(ada, ora, dtype):
    """The bench's 4096-token prompt (batch 1, 32/8 heads, capacity 8192, the
    launch the bench times): token t's outputs are the one-token attention over
    slots 0..t, so the oracle checks sampled tokens one by one -- the first,
    tile and row-tile edges, and the last."""
    B, Hq, Hkv, T, S = 1, 32, 8, 4096, 8192
    say(f"case prefill full size: B={B} Hq={Hq} Hkv={Hkv} T={T} S={S} {dtype}")
    q, k, v = prefill_inputs(B, Hq, Hkv, T, S, dtype, [0], 890)
    scale = 1.0 / math.sqrt(128)
    out = ada.prefill_attn_gqa(q.cuda(), k.cuda(), v.cuda(), None, scale=scale)
    torch.cuda.synchronize()
    got = out.cpu()
    for t in (0, 1, 15, 16, 31, 32, 63, 64, 127, 1000, 2047, 2048, 3071, 4094, 4095):
        want = ora.decode(q[:, :, t, :].contiguous(), k, v, [t + 1], scale).reshape(B, Hq, 1, 128)
        assert_parity(got[:, :, t:t + 1, :], want, dtype, f"token {t}")


def test_prefill_rows_match_decode(ada):
    """Token t of the prefill attends what a one-token decode with
    kv_len = start + t + 1 attends: the two kernels agree within the tolerance."""
    B, Hq, Hkv, T, S = 2, 32, 8, 40, 256
    starts = [0, 50]
    q, k, v = prefill_inputs(B, Hq, Hkv, T, S, "fp16", starts, 850)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = ada.prefill_attn_gqa(qd, kd, vd, torch.tensor(starts, dtype=torch.int32, device="cuda"))
    for t in (0, 1, 17, 39):
        lens = torch.tensor([s + t + 1 for s in starts], dtype=torch.int32, device="cuda")
        dec = ada.decode_attn_gqa(qd[:, :, t, :].contiguous(), kd, vd, lens, max_kv_len=max(starts) + t + 1)
        torch.cuda.synchronize()
        assert_parity(out[:, :, t, :], dec.double().cpu().numpy(), "fp16", f"token {t} vs decode")


def test_prefill_then_decode_pipeline(ada, ora):
    """Prompt append + prefill, then decode steps on the same cache: the
    [ACTIVE-PREFIX] flow (kv_len = T after the prompt, T + i + 1 at step i)."""
    B, Hq, Hkv, T, S = 1, 32, 8, 100, 512
    g = torch.Generator().manual_seed(860)
    q = torch.randn((B, Hq, T, 128), generator=g).half()
    kn = torch.randn((B, Hkv, T, 128), generator=g).half()
    vn = torch.randn((B, Hkv, T, 128), generator=g).half()
    kc = torch.full((B, Hkv, S, 128), float("nan")).half()
    vc = torch.full((B, Hkv, S, 128), float("nan")).half()
    kd, vd = kc.cuda(), vc.cuda()
    ada.prefill_append(kn.cuda(), vn.cuda(), kd, vd)
    out = ada.prefill_attn_gqa(q.cuda(), kd, vd)
    torch.cuda.synchronize()
    kc2, vc2 = ora.prefill_append(kn, vn, kc, vc, [0])
    to16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.float16)
    assert np.array_equal(bits(kd), kc2)
    check_prefill(out, ora.prefill(q, to16(kc2), to16(vc2), [0], 1 / math.sqrt(128)), "fp16", "prompt")
    for i in range(3):
        qs = torch.randn((B, Hq, 128), generator=g).half()
        kns = torch.randn((B, Hkv, 128), generator=g).half()
        vns = torch.randn((B, Hkv, 128), generator=g).half()
        o = ada.decode_step(qs.cuda(), kns.cuda(), vns.cuda(), kd, vd, T + i)
        torch.cuda.synchronize()
        kc2, vc2 = ora.kv_append(kns, vns, to16(kc2), to16(vc2), [T + i])
        assert_parity(o, ora.decode(qs, to16(kc2), to16(vc2), [T + i + 1], 1 / math.sqrt(128)), "fp16", f"step {i}")


def test_prefill_scale_edges(ada, ora):
    """Scale 0 (every visible slot weighs the same: the running mean of the
    value rows) and a negative scale, against the oracle."""
    B, Hq, Hkv, T, S = 2, 8, 2, 70, 200
    for scale, dtype in ((0.0, "fp16"), (-0.09, "bf16")):
        say(f"case prefill scale={scale} {dtype}")
        q, k, v = prefill_inputs(B, Hq, Hkv, T, S, dtype, [0, 60], 870)
        out = ada.prefill_attn_gqa(q.cuda(), k.cuda(), v.cuda(), torch.tensor([0, 60], dtype=torch.int32,
                                                                               device="cuda"), scale=scale)
        torch.cuda.synchronize()
        check_prefill(out, ora.prefill(q, k, v, [0, 60], scale), dtype, f"scale {scale}")
