"""The prefill's per-element error bound (tests/parity.py, prefill_bound)
against a CPU model of the prefill's precision: exact fp64 softmax weights,
rounded once to the 16-bit type (round-to-nearest-even) for both the weighted
sum of value rows and the row sum, fp64 sums, then one RNE rounding of the
output. The bound must hold for every output of the model and stay close to
what the model's worst outputs reach."""
import numpy as np
import pytest
import torch

from parity import prefill_bound

DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def rne(x: np.ndarray, dtype: str) -> np.ndarray:
    return torch.from_numpy(x).to(DT[dtype]).to(torch.float64).numpy()


def model_prefill(q, k, v, lens, scale, dtype):
    """Outputs of the precision model and the exact outputs, [B, H_q, T, D]."""
    B, Hq, T, D = q.shape
    G = Hq // k.shape[1]
    exact = np.zeros((B, Hq, T, D))
    model = np.zeros((B, Hq, T, D))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for t in range(T):
                n = lens[b][t]
                if n == 0:
                    continue
                x = scale * (k[b, g, :n] @ q[b, h, t])
                w = np.exp(x - x.max())
                exact[b, h, t] = w @ v[b, g, :n] / w.sum()
                wr = rne(w, dtype)
                model[b, h, t] = rne(wr @ v[b, g, :n] / wr.sum(), dtype)
    return exact, model


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("scale", [0.0, 0.0883883, 0.5, -0.3])
def test_bound_holds_for_the_precision_model(dtype, scale):
    rng = np.random.default_rng(3 + int(100 * abs(scale)) + (dtype == "bf16"))
    B, Hq, Hkv, T, S, D = 2, 4, 2, 24, 40, 16
    q = rne(rng.standard_normal((B, Hq, T, D)) * 3.0, dtype)
    k = rne(rng.standard_normal((B, Hkv, S, D)) * 3.0, dtype)
    v = rne(rng.standard_normal((B, Hkv, S, D)) * 2.0, dtype)
    starts = [0, 9]
    lens = [[min(S, s + t + 1) for t in range(T)] for s in starts]
    exact, model = model_prefill(q, k, v, lens, scale, dtype)
    bound = prefill_bound(exact, torch.from_numpy(v), lens, dtype)
    err = np.abs(model - exact)
    assert np.all(err <= bound), f"largest error / bound {np.max(err / bound):.3f}"
    # not vacuous: the worst outputs use a good part of their bound
    assert np.max(err / bound) > 0.25


def test_empty_rows_must_be_exact_zeros():
    want = np.zeros((1, 2, 3, 8))
    v = torch.ones((1, 1, 5, 8), dtype=torch.float16)
    b = prefill_bound(want, v, [[0, 0, 0]], "fp16")
    assert np.all(b == 0.0)


def test_half_ulp_term():
    """A single visible slot: the weight term vanishes (v_0 - o = 0) and the
    bound is half an ulp of the output in the 16-bit type."""
    v = torch.tensor([3.0, 5.0, 0.25, -6.0], dtype=torch.float64).reshape(1, 1, 1, 4).to(torch.bfloat16)
    want = v.to(torch.float64).numpy().reshape(1, 1, 1, 4)
    b = prefill_bound(want, v, [[1]], "bf16")[0, 0, 0]
    # bf16 keeps 8 significant bits: half an ulp is 2^(e - 8) for |x| in [2^e, 2^(e+1))
    # (plus the 2^-20 relative allowance for fp32 sums)
    assert np.allclose(b, [2.0 ** -7, 2.0 ** -6, 2.0 ** -10, 2.0 ** -6], rtol=1e-3)


def test_subnormal_outputs_keep_the_fixed_ulp():
    """fp16 outputs below 2^-14 are subnormal: their ulp is 2^-24 whatever
    the value, so half an ulp never falls below 2^-25."""
    v = torch.full((1, 1, 1, 2), 1e-6, dtype=torch.float16)
    want = np.array([[[[1e-6, 3e-7]]]])
    b = prefill_bound(want, v, [[1]], "fp16")
    assert np.all(b >= 2.0 ** -25)
