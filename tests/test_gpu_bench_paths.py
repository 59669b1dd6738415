"""GPU parity of the exact launches bench.py times, at their shapes, through
the C ABI:

* the long-context decode step (the contract line): ada_decode_step with one
  host position, appending at the last of 32768 slots and attending over all
  of them, batch 8, 32/8 heads, bf16, 1 % of key rows x8 -- every batch row
  against the fp64 oracle, the appended rows bit for bit;
* the 36-layer S2-Pro run (fish-speech #1310, "CUDA benchmark"): one library
  step graph over 36 layers, capacity 32768, a 234-token prompt, max_pos 1257
  (20 splits, most of them empty in the early steps), 1024 replays;
* the MiniCPM lockstep sweep (VoxCPM #395, section 6.3): a step graph of 4
  layers, batch 4, capacity 8192, max_pos 8191 (device positions, the
  balanced plan), positions 0 .. 8191.

Unlike the bench, the graph tests write fresh key and value rows before every
replay (so a read of the wrong slot cannot hide behind identical rows) and
check sampled steps and layers against the oracle; every appended cache row
of the checked layers is checked bit for bit at the end.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_parity

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


def bits(t):
    return t.contiguous().view(torch.int16)


def test_long_context_step_every_row(ada, ora):
    wl = W.WORKLOADS["long_context"]
    shp = wl.shape
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    say(f"case long-context decode step: B={B} {Hq}/{Hkv} bf16 S={S}, append at {S - 1} (generating on the GPU)")
    x = W.decode_inputs(shp, [S] * B, W.seed_for(4), device="cuda", tail="random",
                        outlier_p=wl.outlier_p, outlier_scale=wl.outlier_scale)
    kn, vn = W.append_inputs(B, Hkv, D, shp.dtype, W.seed_for(4, 1), device="cuda")
    kc0, vc0 = x["k_cache"].cpu(), x["v_cache"].cpu()
    splits, _ = ada.decode_plan(B, Hq, Hkv, S)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, splits)), "cuda")
    out = torch.empty_like(x["q"])
    ada.decode_step(x["q"], kn, vn, x["k_cache"], x["v_cache"], S - 1, scale=SCALE, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    kc0[:, :, S - 1] = kn.cpu()
    vc0[:, :, S - 1] = vn.cpu()
    assert torch.equal(bits(x["k_cache"][:, :, S - 1].cpu()), bits(kn.cpu()))
    assert torch.equal(bits(x["v_cache"][:, :, S - 1].cpu()), bits(vn.cpu()))
    q = x["q"].cpu()
    del x
    for b in range(B):
        want = ora.decode(q[b:b + 1], kc0[b:b + 1], vc0[b:b + 1], [S], SCALE)
        assert_parity(out[b:b + 1], want, "bf16", f"long-context step, row {b}")


def run_graph_sweep(ada, ora, name, shp, layers, prompt, steps, max_pos, check_steps, check_layers, seed):
    """A library step graph over `layers` layers from position `prompt`, `steps`
    replays with fresh q / k_new / v_new written between them; outputs of
    `check_layers` at `check_steps` against the oracle, appended rows bit for
    bit at the end."""
    B, Hq, Hkv, D, S = shp.batch, shp.n_head, shp.n_kv_head, shp.head_dim, shp.capacity
    dt = W.TORCH_DTYPES[shp.dtype]
    say(f"case {name}: B={B} {Hq}/{Hkv} {shp.dtype} S={S} layers={layers} prompt={prompt} steps={steps} "
        f"max_pos={max_pos}")
    kc = torch.full((layers, B, Hkv, S, D), float("nan"), dtype=dt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    prompt_k, prompt_v = {}, {}
    if prompt > 0:
        for layer in range(layers):
            x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, prompt, shp.dtype), [prompt] * B, seed + layer,
                                device="cuda", tail="random")
            kc[layer, :, :, :prompt] = x["k_cache"]
            vc[layer, :, :, :prompt] = x["v_cache"]
            if layer in check_layers:
                prompt_k[layer], prompt_v[layer] = x["k_cache"].cpu(), x["v_cache"].cpu()
    g = torch.Generator(device="cuda").manual_seed(seed + 1000)
    k_all = torch.randn((steps, layers, B, Hkv, D), generator=g, device="cuda").to(dt)
    v_all = torch.randn((steps, layers, B, Hkv, D), generator=g, device="cuda").to(dt)
    q_buf = torch.randn((layers, B, Hq, D), generator=g, device="cuda").to(dt)
    k_buf = torch.empty((layers, B, Hkv, D), dtype=dt, device="cuda")
    v_buf = torch.empty_like(k_buf)
    out = torch.full((layers, B, Hq, D), float("nan"), dtype=dt, device="cuda")
    pos = torch.full((B,), prompt, dtype=torch.int32, device="cuda")
    splits, _ = ada.decode_plan(B, Hq, Hkv, max_pos + 1)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, D, max(2, splits)), "cuda")
    graph = ada.step_graph([(q_buf[i], k_buf[i], v_buf[i], kc[i], vc[i], out[i]) for i in range(layers)], pos,
                           max_pos, scale=SCALE, workspace=ws)
    try:
        for i in range(steps):
            k_buf.copy_(k_all[i])
            v_buf.copy_(v_all[i])
            if i in check_steps:
                q_buf.copy_(torch.randn((layers, B, Hq, D), generator=g, device="cuda").to(dt))
            graph.launch()
            if i not in check_steps:
                continue
            torch.cuda.synchronize()
            p = prompt + i
            say(f"  {name}: step {i}, position {p}, {splits} splits")
            assert pos.tolist() == [p + 1] * B
            k_hist = k_all[:i + 1].cpu()
            v_hist = v_all[:i + 1].cpu()
            for layer in check_layers:
                kref = torch.full((B, Hkv, p + 1, D), float("nan"), dtype=dt)
                vref = torch.full_like(kref, float("nan"))
                if prompt > 0:
                    kref[:, :, :prompt] = prompt_k[layer]
                    vref[:, :, :prompt] = prompt_v[layer]
                kref[:, :, prompt:] = k_hist[:, layer].permute(1, 2, 0, 3)
                vref[:, :, prompt:] = v_hist[:, layer].permute(1, 2, 0, 3)
                want = ora.decode(q_buf[layer].cpu(), kref, vref, [p + 1] * B, SCALE)
                assert_parity(out[layer], want, shp.dtype, f"{name} step {i} layer {layer}")
        torch.cuda.synchronize()
        for layer in check_layers:
            rows_k = kc[layer, :, :, prompt:prompt + steps].cpu()
            rows_v = vc[layer, :, :, prompt:prompt + steps].cpu()
            assert torch.equal(bits(rows_k), bits(k_all[:, layer].permute(1, 2, 0, 3).cpu())), f"layer {layer} keys"
            assert torch.equal(bits(rows_v), bits(v_all[:, layer].permute(1, 2, 0, 3).cpu())), f"layer {layer} values"
    finally:
        torch.cuda.synchronize()
        graph.close()


def test_s2pro_run_step_graph(ada, ora):
    wl = W.WORKLOADS["s2pro_run"]
    T0, N = wl.prefill, wl.steps
    run_graph_sweep(ada, ora, "S2-Pro step graph", wl.shape, wl.layers, T0, N, T0 + N - 1, {0, 1, 511, N - 1},
                    (0, 17, wl.layers - 1), 30_000)


def test_minicpm_sweep_step_graph(ada, ora):
    shp = W.WORKLOADS["minicpm_stream"].shape
    S = shp.capacity
    run_graph_sweep(ada, ora, "MiniCPM step graph", shp, 4, 0, S, S - 1, {0, 1, 4095, S - 1}, (0, 3), 31_000)


def test_minicpm_ragged_bench_draws(ada, ora):
    """The 64 ragged MiniCPM draws bench.py times (per-row kv_len from the same
    seeds, uniform in [1, 8192]; batch 4, 32/8 heads, bf16): the same call
    with device lengths (the balanced plan) and the heuristic split count,
    against the oracle. The cache is drawn once; each draw's GPU copy gets NaN
    beyond every row's length, so a read past a live prefix shows."""
    shp = W.WORKLOADS["minicpm_stream"].shape
    B, S = shp.batch, shp.capacity
    say(f"case MiniCPM ragged bench draws: B={B} {shp.n_head}/{shp.n_kv_head} {shp.dtype} S={S}, 64 draws")
    x = W.decode_inputs(shp, [S] * B, W.seed_for(3, 70_000), tail="random")
    q, kc, vc = x["q"].cuda(), x["k_cache"].cuda(), x["v_cache"].cuda()
    splits, _ = ada.decode_plan(B, shp.n_head, shp.n_kv_head, S)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, shp.n_head, shp.n_kv_head, 128, max(2, splits)), "cuda")
    out = torch.empty_like(q)
    for d in range(64):
        lens = W.ragged_lengths(B, 1, S, W.seed_for(3, 72_000 + d))
        k_d, v_d = kc.clone(), vc.clone()
        for b, n in enumerate(lens):
            k_d[b, :, n:] = float("nan")
            v_d[b, :, n:] = float("nan")
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
        ada.decode_attn_gqa(q, k_d, v_d, lt, scale=SCALE, out=out, max_kv_len=S, workspace=ws)
        torch.cuda.synchronize()
        want = ora.decode(x["q"], x["k_cache"], x["v_cache"], lens, SCALE)
        assert_parity(out, want, shp.dtype, f"ragged bench draw {d} lens={lens}")
