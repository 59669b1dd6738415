"""The workload shapes and the benchmark's byte model against figures the
pages print (tests/golden/page_figures.json, each entry with its source)."""
import json
from pathlib import Path

import bench
import workloads as W
from parity import TOL

GOLDEN = json.loads((Path(__file__).parent / "golden" / "page_figures.json").read_text())


def test_expanded_full_capacity_bytes():
    """8 KV heads expanded to 32 at full capacity, FP16, K+V: 512 MiB per layer,
    18 GiB over 36 layers (fish-speech #1310, section 1)."""
    g = GOLDEN["s2pro_attention"]
    per_layer = bench.kv_bytes(g["n_head"], g["head_dim"], g["max_seq_len"], elem=2)
    fig = GOLDEN["s2pro_expanded_full_capacity_bytes"]
    assert per_layer == fig["per_layer_mib"] * 2**20
    assert per_layer * g["layers"] == fig["all_layers_gib"] * 2**30
    # the active-prefix, in-place GQA read of the same layer at full length is 4x smaller
    assert bench.kv_bytes(g["n_local_heads"], g["head_dim"], g["max_seq_len"]) * 4 == per_layer


def test_decode_reads_k_and_v_once():
    """Decode cost = reading K and V once: 2 * heads * kv_len * dim elements
    (Cuda-Compute-OSS #343, 'Current limitation')."""
    w = GOLDEN["decode_fastpath_workloads"]
    for n in w["kv_len"]:
        assert bench.kv_bytes(w["heads"], w["dim"], n) == 2 * w["heads"] * n * w["dim"] * 2


def test_projected_per_token_is_36_calls():
    s = GOLDEN["sdpa_microbench"]
    assert abs(s["math_ms_per_call"] * s["layers"] - s["projected_math_ms_36_layers"]) < 0.5
    assert abs(s["efficient_ms_per_call"] * s["layers"] - s["projected_efficient_ms_36_layers"]) < 0.5


def test_workload_shapes_follow_the_pages():
    s2 = GOLDEN["s2pro_attention"]
    tiny = W.WORKLOADS["tiny"].shape
    run = W.WORKLOADS["s2pro_run"]
    for shp in (tiny, run.shape):
        assert (shp.n_head, shp.n_kv_head, shp.head_dim) == (s2["n_head"], s2["n_local_heads"], s2["head_dim"])
    assert run.shape.capacity == s2["max_seq_len"] and run.layers == s2["layers"]
    assert run.prefill == s2["prompt_tokens"] and run.steps == GOLDEN["s2pro_run"]["max_new_tokens"]
    assert run.shape.dtype == GOLDEN["s2pro_run"]["dtype"]
    d = GOLDEN["decode_fastpath_workloads"]
    mha = W.WORKLOADS["mha_sweep"]
    assert mha.kv_lens == tuple(d["kv_len"]) and mha.shape.n_head == mha.shape.n_kv_head == d["heads"]
    assert mha.shape.head_dim == d["dim"] and mha.shape.dtype == d["dtype"]
    m = GOLDEN["minicpm_cache"]
    mc = W.WORKLOADS["minicpm_stream"].shape
    assert (mc.n_kv_head, mc.capacity, mc.head_dim) == (m["kv_heads"], m["max_length"], m["head_dim"])
    assert W.seed_for(2) - 2 == GOLDEN["s2pro_run"]["seed"]


def test_tolerances_at_least_as_strict_as_the_page():
    t = GOLDEN["decode_fastpath_tolerance"]
    for max_abs, rel in TOL.values():
        assert max_abs <= t["abs_max"] and rel <= t["rel_frobenius_max"]
