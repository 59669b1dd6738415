"""Plausible mistakes planted in copies of the oracle source must fail the pins.

Each mutant is a one-place textual change to ``oracle/ada_oracle.c`` (a wrong
head mapping, a dropped term, a flipped sign, a wrong stride, a swapped
operand, a decoder slip). The copy is compiled on the CPU into a temporary
library and every pin of ``oracle_pins`` is run against it; at least one must
fail. This shows the pins would catch such a mistake in the real oracle.
"""
import tempfile

import pytest

import oracle
import oracle_pins

MUTANTS = [
    # grouped-query mapping: tile order instead of repeat_interleave order
    ("head_map_modulo", "const int g = h / group;", "const int g = h % n_kv_head;"),
    # scale dropped from the scores
    ("scale_dropped", "x[j] = scale * dot;", "x[j] = dot;"),
    # sign flipped inside the exponential
    ("exp_sign_flipped", "x[j] = exp(x[j] - m);", "x[j] = exp(m - x[j]);"),
    # max subtraction dropped (overflows on large scores)
    ("max_not_subtracted", "x[j] = exp(x[j] - m);", "x[j] = exp(x[j]);"),
    # normalisation dropped
    ("no_normalisation", "for (int d = 0; d < head_dim; ++d) o[d] /= wsum;", ""),
    # running sum overwritten instead of accumulated
    ("sum_not_accumulated", "wsum += x[j];", "wsum = x[j];"),
    # key row stride wrong (reads overlapping rows)
    ("key_stride", "const uint16_t* krow = kbase + (size_t)j * head_dim;",
     "const uint16_t* krow = kbase + (size_t)j;"),
    # value operand swapped for the key cache
    ("values_from_keys", "v_cache + ((size_t)b * n_kv_head + g)", "k_cache + ((size_t)b * n_kv_head + g)"),
    # query row of the wrong head (KV head index instead of query head)
    ("query_row_index", "const uint16_t* qrow = q + bh * head_dim;",
     "const uint16_t* qrow = q + ((long)b * n_head + g) * head_dim;"),
    # one slot past the active prefix is read
    ("reads_past_prefix", "if (n > capacity) n = capacity;",
     "n = n + 1;\n    if (n > capacity) n = capacity;"),
    # first slot left out of the weighted sum of value rows
    ("first_slot_skipped", "for (int j = 0; j < n; ++j) {\n      const uint16_t* vrow",
     "for (int j = 1; j < n; ++j) {\n      const uint16_t* vrow"),
    # an empty prefix treated as a one-slot prefix
    ("empty_not_zero", "if (n < 0) n = 0;", "if (n < 1) n = 1;"),
    # fp16 decoder slips
    ("f16_fraction_scale", "(double)frac / 1024.0", "(double)frac / 1023.0"),
    ("f16_bias", "expo - 15);", "expo - 14);"),
    ("f16_subnormal", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    # bf16 decoder slips
    ("bf16_exponent_field", "int expo = (bits >> 7) & 0xff;", "int expo = (bits >> 8) & 0xff;"),
    ("bf16_bias", "expo - 127);", "expo - 126);"),
    # append writes slot pos + 1
    ("append_off_by_one", "(((size_t)b * n_kv_head + g) * capacity + p) * head_dim",
     "(((size_t)b * n_kv_head + g) * capacity + p + (p + 1 < capacity)) * head_dim"),
    # prefill: a token sees only the slots before its own position
    ("prefill_off_by_one", "long nl = (long)start[b] + t + 1;", "long nl = (long)start[b] + t;"),
    # prefill: the prompt's first position ignored (top-left causal alignment)
    ("prefill_ignores_start", "long nl = (long)start[b] + t + 1;", "long nl = (long)t + 1;"),
    # prefill: token-major instead of head-major query layout
    ("prefill_query_layout", "const int t = (int)(r % q_len);\n    const int h = (int)((r / q_len) % n_head);",
     "const int h = (int)(r % n_head);\n    const int t = (int)((r / n_head) % q_len);"),
    # prefill: tile head map
    ("prefill_head_map", "const int g = h / group;\n    long nl", "const int g = h % n_kv_head;\n    long nl"),
    # prefill append: rows written one slot late
    ("prefill_append_shift", "long p = (long)start[b] + t;", "long p = (long)start[b] + t + 1;"),
    # prefill append: source row of the wrong token
    ("prefill_append_source", "size_t src = (((size_t)b * n_kv_head + g) * q_len + t) * head_dim;",
     "size_t src = (((size_t)b * n_kv_head + g) * q_len) * head_dim;"),
    # append ignores the out-of-range guard on the low side (writes slot 0)
    ("append_negative_pos", "if (p < 0 || p >= capacity) continue;",
     "if (p >= capacity) continue;\n    if (p < 0) p = 0;"),
]


@pytest.fixture(scope="module")
def source():
    return oracle.SOURCE.read_text()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new):
    assert source.count(old) >= 1, f"mutation site for {name} no longer in the oracle source"
    text = source.replace(old, new, 1)
    with tempfile.TemporaryDirectory(prefix="ada_mutant_") as d:
        lib = oracle.build_from_text(text, d)
        mutant = oracle.Oracle(lib)
        failures = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError, FloatingPointError) as exc:
                failures.append((pin.__name__, str(exc)[:80]))
        assert failures, f"mutant {name} passed every pin"
