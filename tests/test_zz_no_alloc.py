"""GPU test of ada_decode_attn_gqa_noalloc, the decode entry point that
allocates nothing (its split partials live in the library's static
per-device scratch buffer), called through the C ABI.

Each case is checked against the existing entry point, ada_decode_attn_gqa_ex
with a caller-owned workspace and the same split count (same kernels and
plan, so the outputs must agree bit for bit), and against the fp64 oracle
within the decode tolerances. Calls run back to back on one device: a large
one first, then smaller ones that reuse the scratch the first left behind."""
import ctypes
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


def vp(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def noalloc(ada, q, k, v, lens_t, max_kv_len, scale, dtype, out, splits):
    B, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    return ada._lib.ada_decode_attn_gqa_noalloc(vp(q), vp(k), vp(v), vp(lens_t), B, Hq, Hkv, D, S, max_kv_len,
                                                ctypes.c_float(scale), 1 if dtype == "bf16" else 0, vp(out),
                                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), splits)


def run_case(ada, ora, B, Hq, Hkv, S, dtype, lens, seed, splits, device_lens, what):
    say(f"case noalloc {what}: B={B} Hq={Hq} Hkv={Hkv} S={S} {dtype} lens={lens[:8]} splits={splits} "
        f"device_lens={device_lens}")
    x = W.decode_inputs(W.DecodeShape(B, Hq, Hkv, 128, S, dtype), lens, seed, tail="nan")
    d = {k: t.cuda() for k, t in x.items()}
    scale = float(np.float32(1 / math.sqrt(128)))
    if device_lens:
        lens_t, mkl = torch.tensor(lens, dtype=torch.int32, device="cuda"), S
    else:
        assert all(n == lens[0] for n in lens)
        lens_t, mkl = None, lens[0]
    out = torch.full_like(d["q"], float("nan"))
    rc = noalloc(ada, d["q"], d["k_cache"], d["v_cache"], lens_t, mkl, scale, dtype, out, splits)
    assert rc == 0, f"ada_decode_attn_gqa_noalloc returned {rc} ({ada.status_string(rc)})"
    used, _ = ada.decode_plan(B, Hq, Hkv, mkl, splits)
    ws = ada.new_workspace(ada.decode_workspace_bytes(B, Hq, Hkv, 128, max(2, used)), "cuda")
    ref = ada.decode_attn_gqa_ex(d["q"], d["k_cache"], d["v_cache"], lens_t if device_lens else lens[0],
                                 scale=scale, max_kv_len=mkl if device_lens else None, num_splits=splits,
                                 workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{what}: differs from the workspace entry point"
    want = ora.decode(x["q"], x["k_cache"], x["v_cache"], lens, scale)
    assert_parity(out, want, dtype, f"noalloc {what}")
    return used


def test_noalloc_matches_workspace_entry_point(ada, ora):
    # 1. large: the long-context head shape at 8192 slots, ragged device lengths (balanced plan)
    lens = [8192, 1, 5000, 0, 8192, 3333, 7000, 64]
    s1 = run_case(ada, ora, 8, 32, 8, 8192, "bf16", lens, 9100, 0, True, "large ragged")
    assert s1 >= 2, "the first call must use the scratch"
    # 2. smaller, right after it: fewer rows and heads, host length, fp16
    s2 = run_case(ada, ora, 2, 16, 4, 1000, "fp16", [700, 700], 9101, 0, False, "smaller")
    assert s2 >= 2
    # 3. smaller still, a forced split count (MHA heads)
    run_case(ada, ora, 1, 16, 16, 4096, "fp16", [4096], 9102, 32, False, "forced 32 splits")
    # 4. one split: no scratch used at all
    run_case(ada, ora, 1, 32, 8, 200, "bf16", [150], 9103, 1, False, "one split")


def test_noalloc_rejects_over_the_limit(ada):
    """A call whose partials exceed the scratch is refused before any launch."""
    B, Hq, Hkv, S = 64, 64, 8, 4096
    assert ada.decode_workspace_bytes(B, Hq, Hkv, 128, 256) > (4 << 20)
    q = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    k = torch.empty((B, Hkv, 16, 128), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    rc = ada._lib.ada_decode_attn_gqa_noalloc(vp(q), vp(k), vp(k), None, B, Hq, Hkv, 128, 16, 16,
                                              ctypes.c_float(0.1), 0, vp(out),
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), 16)
    assert rc == -12
