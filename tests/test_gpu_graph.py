"""GPU: the graph-captured multi-layer decode step (ada_step_graph_*), called
through the C ABI.

Decode step i after a T-token prompt appends at slot T + i and attends over
T + i + 1 slots ([ACTIVE-PREFIX] section 2; per layer, [FORWARD-STEP]
section 4). The library records every layer's decode step and the position
advance once as a HIP graph; each replay must give, bit for bit, what eager
ada_decode_step (or ada_decode_step_rope) calls with the same max_pos give,
write the same cache rows, advance pos by one, and match the fp64 oracle
within the decode tolerances. Between replays the test rewrites the layers'
query and new-row buffers with eager copies, as a model would.
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


CASES = [
    # name, dtype, B, Hq, Hkv, S, layers, start positions, steps, rotary layers
    ("one row, split plan", "fp16", 1, 32, 8, 2048, 3, [300], 5, ()),
    ("ragged rows, balanced plan, rotary layer", "bf16", 4, 32, 8, 1024, 3, [10, 500, 1019, 63], 4, (1,)),
    ("MHA from an empty cache", "fp16", 2, 16, 16, 512, 2, [0, 255], 3, ()),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_step_graph_replays_equal_eager_steps(ada, ora, case):
    name, dtype, B, Hq, Hkv, S, L, pos0, N, rope_layers = case
    D = 128
    max_pos = max(pos0) + N - 1
    assert max_pos < S
    say(f"case step graph '{name}': {dtype} B={B} Hq={Hq} Hkv={Hkv} S={S} layers={L} pos0={pos0} steps={N}")
    shp = W.DecodeShape(B, Hq, Hkv, D, S, dtype)
    dt = W.TORCH_DTYPES[dtype]
    g_kc, g_vc, e_kc, e_vc = [], [], [], []
    for layer in range(L):
        x = W.decode_inputs(shp, pos0, 4000 + 10 * layer, tail="nan")
        g_kc.append(x["k_cache"].cuda())
        g_vc.append(x["v_cache"].cuda())
        e_kc.append(x["k_cache"].cuda())
        e_vc.append(x["v_cache"].cuda())
    q = [torch.empty((B, Hq, D), dtype=dt, device="cuda") for _ in range(L)]
    kn = [torch.empty((B, Hkv, D), dtype=dt, device="cuda") for _ in range(L)]
    vn = [torch.empty((B, Hkv, D), dtype=dt, device="cuda") for _ in range(L)]
    cs = [torch.empty((B, D), dtype=dt, device="cuda") for _ in range(L)]
    sn = [torch.empty((B, D), dtype=dt, device="cuda") for _ in range(L)]
    g_out = [torch.empty((B, Hq, D), dtype=dt, device="cuda") for _ in range(L)]
    e_out = [torch.empty_like(o) for o in g_out]
    layers = []
    for layer in range(L):
        tup = (q[layer], kn[layer], vn[layer], g_kc[layer], g_vc[layer], g_out[layer])
        layers.append(tup + (cs[layer], sn[layer]) if layer in rope_layers else tup)
    pos_g = torch.tensor(pos0, dtype=torch.int32, device="cuda")
    pos_e = pos_g.clone()
    graph = ada.step_graph(layers, pos_g, max_pos, scale=SCALE)
    try:
        for i in range(N):
            now = [p + i for p in pos0]
            # new inputs for this step, written by eager copies between replays
            for layer in range(L):
                q[layer].copy_(W.randn16((B, Hq, D), dtype, 5000 + 100 * i + layer).cuda())
                k1, v1 = W.append_inputs(B, Hkv, D, dtype, 6000 + 100 * i + layer)
                kn[layer].copy_(k1.cuda())
                vn[layer].copy_(v1.cuda())
                c1, s1 = W.rope_tables(now, D, dtype)
                cs[layer].copy_(c1.cuda())
                sn[layer].copy_(s1.cuda())
            before = [(g_kc[layer].cpu(), g_vc[layer].cpu()) for layer in range(L)] if i in (0, N - 1) else None
            graph.launch()
            for layer in range(L):
                if layer in rope_layers:
                    ada.decode_step_rope(q[layer], kn[layer], vn[layer], cs[layer], sn[layer], e_kc[layer],
                                         e_vc[layer], pos_e, scale=SCALE, out=e_out[layer], max_pos=max_pos)
                else:
                    ada.decode_step(q[layer], kn[layer], vn[layer], e_kc[layer], e_vc[layer], pos_e, scale=SCALE,
                                    out=e_out[layer], max_pos=max_pos)
            pos_e.add_(1)
            torch.cuda.synchronize()
            say(f"  step {i}: positions {now}")
            assert pos_g.tolist() == [p + 1 for p in now], "the graph must advance every position by one"
            for layer in range(L):
                assert torch.equal(g_out[layer], e_out[layer]), f"step {i} layer {layer}: graph != eager step"
                assert torch.equal(bits(g_kc[layer]), bits(e_kc[layer])), f"step {i} layer {layer}: key cache"
                assert torch.equal(bits(g_vc[layer]), bits(e_vc[layer])), f"step {i} layer {layer}: value cache"
                if layer not in rope_layers:
                    for b in range(B):
                        assert torch.equal(bits(g_kc[layer][b, :, now[b]]), bits(kn[layer][b]))
                        assert torch.equal(bits(g_vc[layer][b, :, now[b]]), bits(vn[layer][b]))
            if before is None:
                continue
            for layer in range(L):
                kc0, vc0 = before[layer]
                if layer in rope_layers:
                    want, _, kc1, vc1 = oracle.decode_step_rope(ora, q[layer].cpu(), kn[layer].cpu(), vn[layer].cpu(),
                                                               cs[layer].cpu(), sn[layer].cpu(), kc0, vc0, now,
                                                               SCALE, dtype)
                    assert np.array_equal(bits(g_kc[layer].cpu()).numpy().view(np.uint16), kc1)
                    assert np.array_equal(bits(g_vc[layer].cpu()).numpy().view(np.uint16), vc1)
                else:
                    want = ora.decode(q[layer].cpu(), g_kc[layer].cpu(), g_vc[layer].cpu(), [p + 1 for p in now],
                                      SCALE)
                assert_parity(g_out[layer], want, dtype, f"graph step {i} layer {layer}")
    finally:
        torch.cuda.synchronize()
        graph.close()


def test_step_graph_without_advance_repeats_the_step(ada):
    """advance = False: positions stay, so two replays of the same inputs give
    the same output and write the same slot."""
    B, Hq, Hkv, D, S = 2, 32, 8, 128, 1024
    x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, D, S, "fp16"), [700, 900], 4100, tail="nan")
    kc, vc = x["k_cache"].cuda(), x["v_cache"].cuda()
    q = x["q"].cuda()
    kn, vn = (t.cuda() for t in W.append_inputs(B, Hkv, D, "fp16", 4101))
    out = torch.empty_like(q)
    pos = torch.tensor([700, 900], dtype=torch.int32, device="cuda")
    say("case step graph without advance: B=2 32/8 fp16 pos [700, 900]")
    graph = ada.step_graph([(q, kn, vn, kc, vc, out)], pos, 1000, scale=SCALE, advance=False)
    try:
        graph.launch()
        torch.cuda.synchronize()
        first = out.clone()
        out.zero_()
        graph.launch()
        torch.cuda.synchronize()
        assert pos.tolist() == [700, 900]
        assert torch.equal(out, first)
        ref = ada.decode_step(q, kn, vn, kc.clone(), vc.clone(), pos, scale=SCALE, max_pos=1000)
        torch.cuda.synchronize()
        assert torch.equal(ref, first)
    finally:
        torch.cuda.synchronize()
        graph.close()
