"""GPU parity: libada's HIP kernels against the fp64 CPU oracle, called through
the C ABI (ctypes binding), on seeded synthetic inputs of the pages' shapes.

Pages (cited by title and section):
  [DECODE-FASTPATH] Cuda-Compute-OSS #343, "one-token decode fast path ...".
  [ACTIVE-PREFIX]   fish-speech #1310, "Optimize native AR decoding by
                    attending only to the active KV-cache prefix".
  [FORWARD-STEP]    VoxCPM #395, "MiniCPM4 MiniCPMAttention.forward_step
                    Attention Performance Fix".

Tolerances (tests/parity.py): fp16 max-abs 4e-3, rel-Frobenius 1e-3; bf16
1.6e-2 and 4e-3; every output finite. Cache tails are NaN unless stated, so
any read past kv_len shows up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_parity, compare, to_f64

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1.0 / math.sqrt(128)))


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


def shape(B, Hq, Hkv, S, dtype):
    return W.DecodeShape(B, Hq, Hkv, 128, S, dtype)


def gpu(x):
    return {k: v.cuda() for k, v in x.items()}


def run(ada, ora, shp, lens, seed, *, splits=0, tail="nan", scale=SCALE, max_kv_len=None, what=""):
    say(f"case {what}: B={shp.batch} Hq={shp.n_head} Hkv={shp.n_kv_head} S={shp.capacity} "
        f"{shp.dtype} lens={lens if len(lens) <= 8 else str(lens[:8]) + '...'} splits={splits} seed={seed}")
    x = W.decode_inputs(shp, lens, seed, tail=tail)
    d = gpu(x)
    mkl = max_kv_len if max_kv_len is not None else max(1, min(shp.capacity, max(lens)))
    out = ada.decode_attn_gqa_ex(d["q"], d["k_cache"], d["v_cache"], d["kv_len"], scale=scale,
                                 max_kv_len=mkl, num_splits=splits)
    torch.cuda.synchronize()
    eff = [max(0, min(n, mkl)) for n in lens]
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], eff, scale)
    st = assert_parity(out, want, shp.dtype, what)
    return out, want, x, st


# ---------------------------------------------------------------------------
# The five workloads.


def test_tiny_config(ada, ora):
    """Tiny decode step: batch 1, 32/8 heads, fp16, kv_len 400 in a 2048-slot cache."""
    shp = shape(1, 32, 8, 2048, "fp16")
    for splits in (0, 1, 2, 3, 7, 256):
        run(ada, ora, shp, [400], W.seed_for(0), splits=splits, what=f"tiny splits={splits}")


@pytest.mark.parametrize("kv", [1024, 4096, 8192])
def test_mha_sweep(ada, ora, kv):
    """One-token decode workloads: batch 1, 16 heads (MHA), fp16, kv_len 1024/4096/8192
    ([DECODE-FASTPATH], "Current limitation")."""
    shp = shape(1, 16, 16, 8192, "fp16")
    run(ada, ora, shp, [kv], W.seed_for(1, kv), what=f"mha kv={kv}")
    run(ada, ora, shp, [kv], W.seed_for(1, kv), splits=1, what=f"mha kv={kv} one split")


def test_s2pro_run(ada, ora):
    """S2-Pro-shaped run: 36 layers, 32/8 heads, fp16, capacity 32768, prefill 234
    then 1024 decode steps (append at slot 234+i, attend over 235+i slots);
    parity at sampled (step, layer) pairs ([ACTIVE-PREFIX], "CUDA benchmark" and
    section 2)."""
    wl = W.WORKLOADS["s2pro_run"]
    shp = wl.shape
    L, T0, N = wl.layers, wl.prefill, wl.steps
    last = T0 + N  # 1258 slots ever written
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    dt = W.TORCH_DTYPES[shp.dtype]
    say("case s2pro: generating per-layer K/V")
    rows = [W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, last, shp.dtype), [last], W.seed_for(2, layer),
                            tail="random") for layer in range(L)]
    kc = torch.full((L, B, Hkv, S, D), float("nan"), dtype=dt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    for layer in range(L):
        kc[layer, :, :, :T0] = rows[layer]["k_cache"][:, :, :T0].cuda()
        vc[layer, :, :, :T0] = rows[layer]["v_cache"][:, :, :T0].cuda()
    kg = torch.stack([r["k_cache"] for r in rows]).cuda()  # [L, B, Hkv, last, D]
    vg = torch.stack([r["v_cache"] for r in rows]).cuda()
    qg = W.randn16((N, L, B, Hq, D), shp.dtype, W.seed_for(2, 10_000), device="cuda")
    sample_steps = sorted({0, 1, 2, 63, 64, 65, 511, 512, N - 2, N - 1} | set(range(0, N, 128)))
    sample_layers = (0, 17, L - 1)
    kept = {}
    out = torch.empty((B, Hq, D), dtype=dt, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    say("case s2pro: running 1024 steps x 36 layers")
    for i in range(N):
        pos.fill_(T0 + i)
        lens.fill_(T0 + i + 1)
        for layer in range(L):
            ada.kv_append(kg[layer, :, :, T0 + i].contiguous(), vg[layer, :, :, T0 + i].contiguous(),
                          kc[layer], vc[layer], pos)
            ada.decode_attn_gqa(qg[i, layer], kc[layer], vc[layer], lens, scale=SCALE, out=out,
                                max_kv_len=T0 + i + 1)
            if i in sample_steps and layer in sample_layers:
                kept[(i, layer)] = out.clone()
    torch.cuda.synchronize()
    worst = 0.0
    for (i, layer), got in kept.items():
        n = T0 + i + 1
        want = ora.decode(qg[i, layer].cpu(), rows[layer]["k_cache"][:, :, :n].contiguous(),
                          rows[layer]["v_cache"][:, :, :n].contiguous(), [n], SCALE)
        st = assert_parity(got, want, "fp16", f"s2pro step {i} layer {layer}")
        worst = max(worst, st["rel_fro"])
    say(f"s2pro: {len(kept)} sampled calls, worst rel-Frobenius {worst:.2e}")


def test_minicpm_lockstep_sweep(ada, ora):
    """MiniCPM-style streaming, lockstep: batch 4, 32/8 heads, bf16, capacity 8192;
    position p = 0..8191 appended then attended over p+1 slots for every row
    ([FORWARD-STEP] section 4). Parity at sampled positions."""
    wl = W.WORKLOADS["minicpm_stream"]
    shp = wl.shape
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    say("case minicpm lockstep: generating")
    gen = W.decode_inputs(shp, [S] * B, W.seed_for(3), tail="random")
    kg, vg = gen["k_cache"].cuda(), gen["v_cache"].cuda()
    qg = W.randn16((S, B, Hq, D), shp.dtype, W.seed_for(3, 1), device="cuda")
    kc = torch.full_like(kg, float("nan"))
    vc = torch.full_like(vg, float("nan"))
    out = torch.empty((B, Hq, D), dtype=kg.dtype, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    samples = sorted({0, 1, 2, 63, 64, 127, 128, 4095, 4096, S - 1} | set(range(511, S, 1024)))
    kept = {}
    for p in range(S):
        pos.fill_(p)
        lens.fill_(p + 1)
        ada.kv_append(kg[:, :, p].contiguous(), vg[:, :, p].contiguous(), kc, vc, pos)
        ada.decode_attn_gqa(qg[p], kc, vc, lens, scale=SCALE, out=out, max_kv_len=p + 1)
        if p in samples:
            kept[p] = out.clone()
    torch.cuda.synchronize()
    for p, got in kept.items():
        n = p + 1
        want = ora.decode(qg[p].cpu(), gen["k_cache"][:, :, :n].contiguous(), gen["v_cache"][:, :, :n].contiguous(),
                          [n] * B, SCALE)
        assert_parity(got, want, "bf16", f"minicpm lockstep p={p}")
    say(f"minicpm lockstep: {len(kept)} sampled positions")


def test_minicpm_ragged_draws(ada, ora):
    """MiniCPM-style streaming, ragged: per-row kv_len uniform in [1, 8192]."""
    shp = W.WORKLOADS["minicpm_stream"].shape
    for k in range(12):
        lens = W.ragged_lengths(shp.batch, 1, shp.capacity, W.seed_for(3, 100 + k))
        run(ada, ora, shp, lens, W.seed_for(3, 200 + k), what=f"minicpm ragged draw {k}")


def test_long_context(ada, ora):
    """Long context: batch 8, 32/8 heads, bf16, kv_len 32768 = capacity, 1% of key
    rows scaled x8, device lengths (the balanced plan). Parity on every batch row
    (the oracle computes rows one by one); every output finite."""
    wl = W.WORKLOADS["long_context"]
    shp = wl.shape
    say("case long context: generating on the GPU")
    x = W.decode_inputs(shp, [shp.capacity] * shp.batch, W.seed_for(4), device="cuda", tail="random",
                        outlier_p=wl.outlier_p, outlier_scale=wl.outlier_scale)
    out = ada.decode_attn_gqa(x["q"], x["k_cache"], x["v_cache"], x["kv_len"], scale=SCALE,
                              max_kv_len=shp.capacity)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    for b in range(shp.batch):
        say(f"long context: oracle row {b}")
        want = ora.decode(x["q"][b:b + 1].cpu(), x["k_cache"][b:b + 1].cpu(), x["v_cache"][b:b + 1].cpu(),
                          [shp.capacity], SCALE)
        assert_parity(out[b:b + 1], want, "bf16", f"long context row {b}")


def test_large_capacity(ada, ora):
    """Caches of 2^22 slots per (batch row, KV head), 3 GiB each for K and V:
    slot offsets past 2^31 bytes, the heuristic's cap of 256 splits
    (16384-slot ranges, so the combine merges 8 batches of 32 partials), a
    ragged short row beside full ones (device lengths: the balanced plan), and
    a decode step with per-row positions at the end. Inputs drawn on the GPU;
    the oracle computes every row."""
    S = 1 << 22
    B = 3
    shp = shape(B, 2, 1, S, "bf16")
    lens = [S, 77, S - 5]
    say(f"case large capacity: S={S} lens={lens}: generating on the GPU")
    x = W.decode_inputs(shp, lens, 7300, device="cuda", tail="nan")
    assert ada.decode_num_splits(B, 2, 1, S) == 256
    out = ada.decode_attn_gqa(x["q"], x["k_cache"], x["v_cache"], x["kv_len"], scale=SCALE, max_kv_len=S)
    torch.cuda.synchronize()
    q, kc, vc = x["q"].cpu(), x["k_cache"].cpu(), x["v_cache"].cpu()
    assert_parity(out, ora.decode(q, kc, vc, lens, SCALE), "bf16", "large capacity")
    pos = [S - 1, 77, S - 5]
    kn, vn = W.append_inputs(B, 1, 128, "bf16", 7301)
    pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    step = ada.decode_step(x["q"], kn.cuda(), vn.cuda(), x["k_cache"], x["v_cache"], pos_t, scale=SCALE)
    torch.cuda.synchronize()
    for b, p_ in enumerate(pos):
        kc[b, :, p_] = kn[b]
        vc[b, :, p_] = vn[b]
        got_k = x["k_cache"][b, :, p_].cpu()
        assert torch.equal(got_k.view(torch.int16), kn[b].view(torch.int16)), f"key row of batch row {b}"
    assert_parity(step, ora.decode(q, kc, vc, [p_ + 1 for p_ in pos], SCALE), "bf16", "large capacity step")


# ---------------------------------------------------------------------------
# Grouped-query sizes, ragged batches and edges.


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8])
def test_group_sizes(ada, ora, dtype, group):
    for hkv in (1, 3):
        lens = W.ragged_lengths(3, 1, 700, 500 + group * 10 + hkv)
        run(ada, ora, shape(3, group * hkv, hkv, 777, dtype), lens, 600 + group, what=f"G={group} Hkv={hkv}")


def test_ragged_batch_edges(ada, ora):
    lens = [0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000]
    out, want, _, _ = run(ada, ora, shape(len(lens), 8, 2, 1000, "bf16"), lens, 701, what="ragged edges")
    assert torch.count_nonzero(out[0]) == 0, "kv_len 0 must give a zero row"
    for splits in (1, 2, 5, 16):
        run(ada, ora, shape(len(lens), 8, 2, 1000, "fp16"), lens, 702, splits=splits, what=f"ragged s={splits}")


def test_all_rows_empty(ada, ora):
    out, _, _, _ = run(ada, ora, shape(2, 8, 2, 64, "fp16"), [0, 0], 703, max_kv_len=64, what="all empty")
    assert torch.count_nonzero(out) == 0


def test_kv_len_one_returns_v0_exactly(ada):
    """Position 0: softmax over one slot is the identity, out = v[0] exactly
    ([FORWARD-STEP] section 3)."""
    for dtype in ("fp16", "bf16"):
        shp = shape(3, 32, 8, 128, dtype)
        x = gpu(W.decode_inputs(shp, [1, 1, 1], 704, tail="nan"))
        for splits in (0, 1, 4):
            out = ada.decode_attn_gqa_ex(x["q"], x["k_cache"], x["v_cache"], x["kv_len"], scale=SCALE,
                                         max_kv_len=128, num_splits=splits)
            want = x["v_cache"][:, :, 0, :].repeat_interleave(4, dim=1)
            assert torch.equal(out, want), f"kv_len 1 must return v[0] exactly ({dtype}, splits {splits})"


def test_equal_scores_give_mean(ada):
    """Scale 0 (and identical keys) give the plain mean of the live value rows."""
    shp = shape(2, 8, 2, 300, "fp16")
    lens = [300, 37]
    x = W.decode_inputs(shp, lens, 705, tail="nan")
    d = gpu(x)
    vd = x["v_cache"].to(torch.float64)
    want = np.stack([vd[b, :, :n].mean(dim=1).repeat_interleave(4, dim=0).numpy() for b, n in enumerate(lens)])
    out = ada.decode_attn_gqa(d["q"], d["k_cache"], d["v_cache"], d["kv_len"], scale=0.0, max_kv_len=300)
    assert_parity(out, want, "fp16", "scale 0")
    k_same = d["k_cache"].clone()
    k_same[:] = d["k_cache"][:, :, :1]
    out = ada.decode_attn_gqa(d["q"], k_same, d["v_cache"], d["kv_len"], scale=SCALE, max_kv_len=300)
    assert_parity(out, want, "fp16", "identical keys")


def test_split_invariance_and_determinism(ada, ora):
    shp = shape(2, 32, 8, 4096, "bf16")
    lens = [4096, 2999]
    x = W.decode_inputs(shp, lens, 706, tail="nan")
    d = gpu(x)
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], lens, SCALE)
    outs = {}
    for splits in (1, 2, 3, 7, 16, 64, 256, 0):
        o1 = ada.decode_attn_gqa_ex(d["q"], d["k_cache"], d["v_cache"], d["kv_len"], scale=SCALE,
                                    max_kv_len=4096, num_splits=splits)
        o2 = ada.decode_attn_gqa_ex(d["q"], d["k_cache"], d["v_cache"], d["kv_len"], scale=SCALE,
                                    max_kv_len=4096, num_splits=splits)
        assert torch.equal(o1, o2), f"not deterministic at {splits} splits"
        assert_parity(o1, want, "bf16", f"splits {splits}")
        outs[splits] = to_f64(o1)
    spread = max(np.max(np.abs(a - outs[1])) for a in outs.values())
    assert spread <= 1.6e-2


def test_workspace_reuse_across_split_counts(ada, ora):
    """One cached workspace serves calls with different split counts in turn
    (it needs no preparation: every partial a combine reads is written by the
    partial launch before it)."""
    shp = shape(4, 32, 8, 2048, "fp16")
    for k, splits in enumerate((7, 3, 0, 2, 31, 0, 1, 5)):
        lens = W.ragged_lengths(4, 1, 2048, 800 + k)
        run(ada, ora, shp, lens, 900 + k, splits=splits, what=f"reuse {k}")


def test_max_kv_len_clamps_device_lengths(ada, ora):
    shp = shape(3, 16, 4, 512, "bf16")
    lens = [500, 300, 100]
    x = W.decode_inputs(shp, lens, 707, tail="nan")
    d = gpu(x)
    out = ada.decode_attn_gqa(d["q"], d["k_cache"], d["v_cache"], d["kv_len"], scale=SCALE, max_kv_len=200)
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], [200, 200, 100], SCALE)
    assert_parity(out, want, "bf16", "max_kv_len clamp")
    lens_big = torch.tensor([10_000, -3, 512], dtype=torch.int32, device="cuda")
    x2 = W.decode_inputs(shp, [512, 512, 512], 708, tail="random")
    d2 = gpu(x2)
    out = ada.decode_attn_gqa(d2["q"], d2["k_cache"], d2["v_cache"], lens_big, scale=SCALE)
    want = ora.decode(x2["q"], x2["k_cache"], x2["v_cache"], [512, 0, 512], SCALE)
    assert_parity(out, want, "bf16", "capacity clamp")


def test_unaligned_lengths_and_capacity(ada, ora):
    for S, lens in ((1000, [999]), (33, [33, 1]), (4097, [4097, 4096, 17])):
        run(ada, ora, shape(len(lens), 8, 1, S, "fp16"), lens, 709 + S, what=f"S={S}")


def test_large_scores_stay_finite(ada, ora):
    shp = shape(2, 8, 2, 256, "bf16")
    x = W.decode_inputs(shp, [256, 99], 710, tail="nan")
    x["k_cache"] = (x["k_cache"].float() * 16).to(torch.bfloat16)
    d = gpu(x)
    out = ada.decode_attn_gqa(d["q"], d["k_cache"], d["v_cache"], d["kv_len"], scale=SCALE, max_kv_len=256)
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], [256, 99], SCALE)
    assert_parity(out, want, "bf16", "large scores")


def test_four_dim_query_and_output(ada, ora):
    shp = shape(2, 32, 8, 512, "fp16")
    x = W.decode_inputs(shp, [512, 200], 711, tail="nan")
    d = gpu(x)
    q4 = d["q"][:, :, None, :].contiguous()
    out = ada.decode_attn_gqa(q4, d["k_cache"], d["v_cache"], [512, 200], scale=SCALE)
    assert out.shape == (2, 32, 1, 128)
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], [512, 200], SCALE)
    assert_parity(out, want, "fp16", "4-d query")


# ---------------------------------------------------------------------------
# In-place append.


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_kv_append_bit_exact(ada, ora, dtype):
    B, Hkv, S, D = 5, 8, 300, 128
    x = W.decode_inputs(W.DecodeShape(B, 32, Hkv, D, S, dtype), [S] * B, 712, tail="random")
    kn, vn = W.append_inputs(B, Hkv, D, dtype, 713)
    pos = [0, 299, -1, 300, 150]
    kc, vc = x["k_cache"].cuda(), x["v_cache"].cuda()
    ada.kv_append(kn.cuda(), vn.cuda(), kc, vc, torch.tensor(pos, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    want_k, want_v = ora.kv_append(kn, vn, x["k_cache"], x["v_cache"], pos)
    got_k = kc.cpu().view(torch.int16).numpy().view(np.uint16)
    got_v = vc.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


def test_append_then_decode_step(ada, ora):
    """One forward step as the pages run it: append at position_id, attend over
    position_id + 1 slots ([FORWARD-STEP] section 4)."""
    B, Hq, Hkv, D, S = 2, 32, 8, 128, 1024
    p = 700
    x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, S, "bf16"), [p] * B, 714, tail="nan")
    kn, vn = W.append_inputs(B, Hkv, D, "bf16", 715)
    d = gpu(x)
    ada.kv_append(kn.cuda(), vn.cuda(), d["k_cache"], d["v_cache"], [p] * B)
    out = ada.decode_attn_gqa(d["q"], d["k_cache"], d["v_cache"], [p + 1] * B, scale=SCALE)
    kc, vc = ora.kv_append(kn, vn, x["k_cache"], x["v_cache"], [p] * B)
    kc_t = torch.from_numpy(kc.view(np.int16)).view(torch.bfloat16)
    vc_t = torch.from_numpy(vc.view(np.int16)).view(torch.bfloat16)
    want = ora.decode(x["q"], kc_t, vc_t, [p + 1] * B, SCALE)
    assert_parity(out, want, "bf16", "append then decode")


# ---------------------------------------------------------------------------
# The two halves: partial + combine, and partials of separate key ranges.


def test_partial_then_combine_equals_decode(ada, ora):
    shp = shape(3, 32, 8, 3000, "bf16")
    lens = [3000, 1, 1777]
    x = gpu(W.decode_inputs(shp, lens, 716, tail="nan"))
    for splits in (1, 5, 0):
        ws, used = ada.decode_partial(x["q"], x["k_cache"], x["v_cache"], x["kv_len"], scale=SCALE,
                                      max_kv_len=3000, num_splits=splits)
        out = torch.empty_like(x["q"])
        ada.decode_combine(ws, used, out, n_kv_head=8)
        ref = ada.decode_attn_gqa_ex(x["q"], x["k_cache"], x["v_cache"], x["kv_len"], scale=SCALE,
                                     max_kv_len=3000, num_splits=splits)
        if used > 1 and splits > 0:  # same forced plan: bit for bit
            assert torch.equal(out, ref), f"partial+combine differs from the decode call at {used} splits"
        else:
            # one split: the decode call writes directly, the combine divides once more;
            # heuristic count with device lengths: the decode call shares the workgroups
            # among the rows by length (balanced plan), the explicit partial keeps one
            # range plan per row -- the same keys, split differently
            assert_parity(out, to_f64(ref), "bf16", f"partial+combine vs decode call, splits={splits}")
            assert_parity(out, ora.decode(x["q"].cpu(), x["k_cache"].cpu(), x["v_cache"].cpu(), lens, SCALE),
                          "bf16", "partial+combine vs oracle")


def test_key_ranges_merged_by_combine(ada, ora):
    """Key ranges attended separately (as shards of a longer cache would be)
    and merged once: partials concatenated along the split axis, one combine.
    Equals attention over the whole prefix."""
    B, Hq, Hkv, S = 2, 32, 8, 6000
    shp = shape(B, Hq, Hkv, S, "fp16")
    lens = [6000, 4500]
    x = W.decode_inputs(shp, lens, 717, tail="nan")
    cut = 2500
    d = gpu(x)
    shard_a = (d["k_cache"][:, :, :cut].contiguous(), d["v_cache"][:, :, :cut].contiguous(), [cut, cut])
    shard_b = (d["k_cache"][:, :, cut:].contiguous(), d["v_cache"][:, :, cut:].contiguous(),
               [n - cut for n in lens])
    parts = []
    for k, v, ln in (shard_a, shard_b):
        ws, used = ada.decode_partial(d["q"], k, v, ln, scale=SCALE, max_kv_len=max(ln), num_splits=3)
        parts.append((ws, used))
    total = sum(u for _, u in parts)
    lay = ada.workspace_layout(B, Hq, total)
    merged = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    ml_row = lay["rows_per_split"] * 8
    acc_row = lay["rows_per_split"] * 128 * 4
    s0 = 0
    for ws, used in parts:
        own = ada.workspace_layout(B, Hq, used)
        merged[lay["ml_offset"] + s0 * ml_row: lay["ml_offset"] + (s0 + used) * ml_row] = \
            ws[own["ml_offset"]: own["ml_offset"] + used * ml_row]
        merged[lay["acc_offset"] + s0 * acc_row: lay["acc_offset"] + (s0 + used) * acc_row] = \
            ws[own["acc_offset"]: own["acc_offset"] + used * acc_row]
        s0 += used
    out = torch.empty_like(d["q"])
    ada.decode_combine(merged, total, out, n_kv_head=Hkv)
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], lens, SCALE)
    assert_parity(out, want, "fp16", "key ranges merged")


def test_lockstep_lengths_from_the_host(ada, ora):
    """One host-side position for the whole batch ([ACTIVE-PREFIX] section 2:
    the length comes from a host int, no device read): NULL device lengths."""
    shp = shape(4, 32, 8, 5000, "bf16")
    for n, splits in ((4321, 0), (1, 0), (700, 3), (5000, 1)):
        x = W.decode_inputs(shp, [n] * 4, 718 + n, tail="nan")
        d = gpu(x)
        out = ada.decode_attn_gqa_ex(d["q"], d["k_cache"], d["v_cache"], n, scale=SCALE, num_splits=splits)
        out2 = ada.decode_attn_gqa_ex(d["q"], d["k_cache"], d["v_cache"], None, scale=SCALE, max_kv_len=n,
                                      num_splits=splits)
        assert torch.equal(out, out2)
        want = ora.decode(x["q"], x["k_cache"], x["v_cache"], [n] * 4, SCALE)
        assert_parity(out, want, "bf16", f"lockstep n={n}")
    x = gpu(W.decode_inputs(shp, [0] * 4, 719, tail="nan"))
    out = ada.decode_attn_gqa(x["q"], x["k_cache"], x["v_cache"], 0, scale=SCALE)
    assert torch.count_nonzero(out) == 0


# ---------------------------------------------------------------------------
# The whole step in one call.


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_decode_step_equals_append_then_decode(ada, ora, dtype):
    """ada_decode_step = ada_kv_append + ada_decode_attn_gqa with kv_len = pos + 1,
    bit for bit, for lockstep and per-row positions ([FORWARD-STEP] section 4)."""
    B, Hq, Hkv, D, S = 4, 32, 8, 128, 3000
    for k, (pos, splits) in enumerate((([2999] * 4, 0), ([1234] * 4, 7), ([0, 5, 2999, 1500], 0),
                                        ([-1, 3000, 77, 2000], 3), ([0] * 4, 1))):
        say(f"case decode step {dtype} pos={pos} splits={splits}")
        # finite slots: those before the new row; a position past the cache leaves it whole
        lens = [S if p >= S else max(0, p) for p in pos]
        x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, S, dtype), lens, 720 + k, tail="nan")
        kn, vn = W.append_inputs(B, Hkv, D, dtype, 740 + k)
        d1, d2 = gpu(x), gpu(x)
        kn_d, vn_d = kn.cuda(), vn.cuda()
        pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
        mp = max(0, min(S - 1, max(pos)))
        fused = ada.decode_step(d1["q"], kn_d, vn_d, d1["k_cache"], d1["v_cache"], pos, scale=SCALE,
                                num_splits=splits)
        ada.kv_append(kn_d, vn_d, d2["k_cache"], d2["v_cache"], pos_t)
        lens_t = torch.tensor([p + 1 if p >= 0 else 0 for p in pos], dtype=torch.int32, device="cuda")
        ref = ada.decode_attn_gqa_ex(d2["q"], d2["k_cache"], d2["v_cache"], lens_t, scale=SCALE,
                                     max_kv_len=mp + 1, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(d1["k_cache"].view(torch.int16), d2["k_cache"].view(torch.int16))
        assert torch.equal(d1["v_cache"].view(torch.int16), d2["v_cache"].view(torch.int16))
        assert torch.equal(fused, ref), "decode_step differs from append + decode"
        kc, vc = ora.kv_append(kn, vn, x["k_cache"], x["v_cache"], pos)
        to16 = lambda a: torch.from_numpy(a.view(np.int16)).view(W.TORCH_DTYPES[dtype])
        eff = [min(p, mp) + 1 if p >= 0 else 0 for p in pos]
        want = ora.decode(x["q"], to16(kc), to16(vc), eff, SCALE)
        assert_parity(fused, want, dtype, f"decode step pos={pos}")


@pytest.mark.parametrize("rope", [False, True])
def test_decode_step_positions_past_the_host_bound(ada, ora, rope):
    """Device positions beyond max_pos: the row is still written at slot pos[b]
    (inside the cache) and the row attends over max_pos + 1 slots; negative
    positions write nothing and give zeros; positions past the cache write
    nothing. Equal, bit for bit, to the append (or rotary append) followed by
    the decode with kv_len = min(pos, max_pos) + 1, for per-row, balanced and
    one-split plans. The extreme int32 positions take the same rules (the
    largest attends over max_pos + 1 slots: pos + 1 must not wrap)."""
    B, Hq, Hkv, D, S, dtype = 7, 32, 8, 128, 2048, "bf16"
    max_pos = 1000
    # at, past the bound (twice), negative, past the cache, int32 extremes
    pos = [1000, 1500, 2047, -1, 2048, 2**31 - 1, -2**31]
    for k, splits in enumerate((0, 1, 3)):
        say(f"case decode step past max_pos rope={rope} pos={pos} max_pos={max_pos} splits={splits}")
        lens = [min(S, max(0, p)) for p in pos]
        x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, S, dtype), lens, 760 + k, tail="nan")
        kn, vn = W.append_inputs(B, Hkv, D, dtype, 770 + k)
        d1, d2 = gpu(x), gpu(x)
        kn_d, vn_d = kn.cuda(), vn.cuda()
        pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
        eff = torch.tensor([min(p, max_pos) + 1 if p >= 0 else 0 for p in pos], dtype=torch.int32, device="cuda")
        if rope:
            cos, sin = (t.cuda() for t in W.rope_tables([max(0, p) for p in pos], D, dtype))
            fused = ada.decode_step_rope(d1["q"], kn_d, vn_d, cos, sin, d1["k_cache"], d1["v_cache"], pos_t,
                                         scale=SCALE, max_pos=max_pos, num_splits=splits)
            q_rot = ada.rope_kv_append(d2["q"], kn_d, vn_d, cos, sin, d2["k_cache"], d2["v_cache"], pos_t)
        else:
            fused = ada.decode_step(d1["q"], kn_d, vn_d, d1["k_cache"], d1["v_cache"], pos_t, scale=SCALE,
                                    max_pos=max_pos, num_splits=splits)
            ada.kv_append(kn_d, vn_d, d2["k_cache"], d2["v_cache"], pos_t)
            q_rot = d2["q"]
        ref = ada.decode_attn_gqa_ex(q_rot, d2["k_cache"], d2["v_cache"], eff, scale=SCALE,
                                     max_kv_len=max_pos + 1, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(d1["k_cache"].view(torch.int16), d2["k_cache"].view(torch.int16)), "key rows differ"
        assert torch.equal(d1["v_cache"].view(torch.int16), d2["v_cache"].view(torch.int16)), "value rows differ"
        assert torch.equal(fused, ref), "decode step differs from append + decode"
        assert torch.count_nonzero(fused[3]) == 0, "a negative position must give a zero row"
        assert torch.count_nonzero(fused[6]) == 0, "a negative position must give a zero row"
        assert torch.count_nonzero(fused[5]) > 0, "the largest position attends over max_pos + 1 slots"
        if not rope:
            kc, vc = ora.kv_append(kn, vn, x["k_cache"], x["v_cache"], pos)
            to16 = lambda a: torch.from_numpy(a.view(np.int16)).view(W.TORCH_DTYPES[dtype])
            want = ora.decode(x["q"], to16(kc), to16(vc), eff.tolist(), SCALE)
            assert_parity(fused, want, dtype, f"decode step past max_pos splits={splits}")


def test_decode_step_position_zero_returns_new_value(ada):
    """Position 0: the only slot is the new one, so out = v_new exactly."""
    x = gpu(W.decode_inputs(shape(2, 16, 4, 64, "bf16"), [0, 0], 760, tail="nan"))
    kn, vn = W.append_inputs(2, 4, 128, "bf16", 761)
    out = ada.decode_step(x["q"], kn.cuda(), vn.cuda(), x["k_cache"], x["v_cache"], 0, scale=SCALE)
    assert torch.equal(out, vn.cuda().repeat_interleave(4, dim=1))


def test_graph_replayed_steps_match_eager(ada, ora):
    """A captured multi-layer decode step with a device-side position increment,
    replayed several times with eager work and synchronisations in between:
    every replay equals the same steps run eagerly, bit for bit, and the first
    matches the oracle."""
    L, B, Hq, Hkv, D, S, T0 = 3, 2, 32, 8, 128, 1024, 300
    dt = torch.float16
    xs = [W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, S, "fp16"), [T0] * B, 770 + l, tail="nan") for l in range(L)]
    new = [W.append_inputs(B, Hkv, D, "fp16", 780 + l) for l in range(L)]
    kg = torch.stack([x["k_cache"] for x in xs]).cuda()
    vg = torch.stack([x["v_cache"] for x in xs]).cuda()
    ke, ve = kg.clone(), vg.clone()
    qg = torch.stack([x["q"] for x in xs]).cuda()
    kn = torch.stack([n[0] for n in new]).cuda()
    vn = torch.stack([n[1] for n in new]).cuda()
    out_g = torch.empty((L, B, Hq, D), dtype=dt, device="cuda")
    out_e = torch.empty_like(out_g)
    pos = torch.full((B,), T0, dtype=torch.int32, device="cuda")
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, 64), torch.device("cuda"))

    def step(kc, vc, out, p, max_pos):
        for l in range(L):
            ada.decode_step(qg[l], kn[l], vn[l], kc[l], vc[l], p, scale=SCALE, out=out[l], max_pos=max_pos,
                            workspace=ws)

    def graph_step():
        step(kg, vg, out_g, pos, S - 1)
        pos.add_(1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    kg.copy_(ke)
    vg.copy_(ve)
    pos.fill_(T0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_step()
    torch.cuda.synchronize()
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        _ = (qg.float() * 2).sum()  # unrelated eager work between replays
        pos_e = torch.full((B,), T0 + r, dtype=torch.int32, device="cuda")
        step(ke, ve, out_e, pos_e, S - 1)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {r} differs from the eager step"
        assert torch.equal(kg.view(torch.int16), ke.view(torch.int16)), f"replay {r}: key caches differ"
        if r == 0:
            for l in range(L):
                kc, vc = ora.kv_append(new[l][0], new[l][1], xs[l]["k_cache"], xs[l]["v_cache"], [T0] * B)
                to16 = lambda a: torch.from_numpy(a.view(np.int16)).view(dt)
                want = ora.decode(xs[l]["q"], to16(kc), to16(vc), [T0 + 1] * B, SCALE)
                assert_parity(out_g[l], want, "fp16", f"graph layer {l}")


def test_balanced_plan_for_device_lengths(ada, ora):
    """Device-side lengths with 2..64 rows use the balanced split plan (each KV
    head's workgroups shared among the rows by length): ragged, empty and
    clamped rows, a single long row among empty ones, 64 rows, and 65 rows
    (the per-row plan again); decode steps with per-row positions too."""
    cases = [
        (shape(4, 32, 8, 8192, "bf16"), [8192, 17, 0, 5000], "ragged with an empty row"),
        (shape(8, 32, 8, 4096, "fp16"), [0, 0, 0, 4096, 0, 0, 0, 0], "one long row"),
        (shape(8, 16, 16, 2048, "fp16"), [0] * 8, "all empty"),
        (shape(64, 8, 2, 512, "bf16"), [int(x) for x in np.random.default_rng(5).integers(0, 513, 64)], "64 rows"),
        (shape(65, 8, 2, 256, "fp16"), [int(x) for x in np.random.default_rng(6).integers(1, 257, 65)], "65 rows"),
        (shape(3, 32, 8, 300, "bf16"), [300, 299, 1], "short rows"),
    ]
    for k, (shp, lens, what) in enumerate(cases):
        run(ada, ora, shp, lens, 980 + k, splits=0, what=f"balanced {what}")
    # decode steps with per-row positions (balanced), out-of-range positions included
    B, Hq, Hkv, D, S = 6, 32, 8, 128, 4096
    pos = [4095, 10, -1, 2000, 4096, 0]
    say(f"case balanced decode step pos={pos}")
    lens = [S if p >= S else max(0, p) for p in pos]
    x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, S, "bf16"), lens, 990, tail="nan")
    kn, vn = W.append_inputs(B, Hkv, D, "bf16", 991)
    d = gpu(x)
    out = ada.decode_step(d["q"], kn.cuda(), vn.cuda(), d["k_cache"], d["v_cache"],
                          torch.tensor(pos, dtype=torch.int32, device="cuda"), scale=SCALE)
    torch.cuda.synchronize()
    kc, vc = ora.kv_append(kn, vn, x["k_cache"], x["v_cache"], pos)
    to16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    eff = [min(p, S - 1) + 1 if p >= 0 else 0 for p in pos]
    assert_parity(out, ora.decode(x["q"], to16(kc), to16(vc), eff, SCALE), "bf16", "balanced decode step")
    assert np.array_equal(d["k_cache"].cpu().view(torch.int16).numpy().view(np.uint16), kc)
