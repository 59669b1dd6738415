"""The rotary oracle against its pins, and planted mistakes against the same pins.

Each mutant is a one-place textual change to ``oracle/rope.py`` (a flipped
sign, a wrong partner element, swapped tables, a wrong table index, a
rounding or decoder slip). The changed source is loaded as a fresh module and
every pin of ``rope_pins`` is run against it; at least one must fail.
"""
import types

import pytest

import oracle.rope as rope_oracle
import rope_pins


@pytest.mark.parametrize("pin", rope_pins.ALL_PINS, ids=[p.__name__ for p in rope_pins.ALL_PINS])
def test_rope_pin(pin):
    pin(rope_oracle)


MUTANTS = [
    ("first_half_sign", "out.append(x[i] * cos[i] - x[i + h] * sin[i])", "out.append(x[i] * cos[i] + x[i + h] * sin[i])"),
    ("second_half_sign", "out.append(x[i] * cos[i] + x[i - h] * sin[i])", "out.append(x[i] * cos[i] - x[i - h] * sin[i])"),
    ("adjacent_partner", "out.append(x[i] * cos[i] - x[i + h] * sin[i])", "out.append(x[i] * cos[i] - x[(i + 1) % d] * sin[i])"),
    ("tables_swapped", "out.append(x[i] * cos[i] - x[i + h] * sin[i])", "out.append(x[i] * sin[i] - x[i + h] * cos[i])"),
    ("partner_table_index", "out.append(x[i] * cos[i] + x[i - h] * sin[i])", "out.append(x[i] * cos[i] + x[i - h] * sin[i - h])"),
    ("ties_away", "pick = bits[j - 1] if bits[j - 1] % 2 == 0 else bits[j]", "pick = bits[j]"),
    ("ties_down", "pick = bits[j - 1] if bits[j - 1] % 2 == 0 else bits[j]", "pick = bits[j - 1]"),
    ("truncation", "if below < above:", "if True:"),
    ("overflow_threshold", "if mag >= top + top_ulp / 2:", "if mag > top + top_ulp / 2:"),
    ("f16_fraction", "(1.0 + frac / 1024.0)", "(1.0 + frac / 1023.0)"),
    ("f16_bias", "2.0 ** (expo - 15)", "2.0 ** (expo - 14)"),
    ("bf16_bias", "2.0 ** (expo - 127)", "2.0 ** (expo - 126)"),
    ("bf16_fraction_bits", "frac = bits & 0x7F", "frac = bits & 0x3F"),
    ("sign_dropped", "sign = 0x8000 if value < 0 else 0", "sign = 0"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_rope_mutant_is_caught(name, old, new):
    source = open(rope_oracle.__file__).read()
    assert source.count(old) >= 1, f"mutation site for {name} no longer in the rotary oracle"
    mutant = types.ModuleType(f"rope_mutant_{name}")
    exec(compile(source.replace(old, new, 1), f"<mutant {name}>", "exec"), mutant.__dict__)
    failures = []
    for pin in rope_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, ZeroDivisionError, IndexError, OverflowError) as exc:
            failures.append((pin.__name__, str(exc)[:80]))
    assert failures, f"mutant {name} passed every pin"


def test_step_with_identity_tables_is_the_plain_step():
    """With cos = 1 and sin = 0 the rotary step is append + decode of the unrotated rows."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    ora = oracle.load()
    shape = W.DecodeShape(2, 8, 2, 128, 64, "bf16")
    x = W.decode_inputs(shape, [40, 64], seed=5, tail="zero")
    k_new, v_new = W.append_inputs(2, 2, 128, "bf16", seed=6)
    pos = [39, 80]  # the second is outside the 64-slot cache: nothing written, all 64 slots attended
    ones = torch.full((2, 128), 1.0, dtype=torch.bfloat16)
    zeros = torch.zeros((2, 128), dtype=torch.bfloat16)
    out, q_rot, kc, vc = oracle.decode_step_rope(ora, x["q"], k_new, v_new, ones, zeros,
                                                 x["k_cache"], x["v_cache"], pos, 0.0884, "bf16")
    kc2, vc2 = ora.kv_append(k_new, v_new, x["k_cache"], x["v_cache"], pos)
    want = ora.decode(x["q"], kc2, vc2, [40, 64], 0.0884)
    assert np.array_equal(q_rot, oracle._bits(x["q"]))
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)
    assert np.array_equal(out, want)
