"""Host side of the C ABI, on the CPU: the library loads, exports every
function ``include/ada.h`` declares, and rejects every invalid argument
before any HIP call (no GPU is touched by these tests)."""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "ada.h"


@pytest.fixture(scope="module")
def ada():
    lib_path = ROOT / "autoregressive_decode_attention_amd" / "libada.so"
    if not lib_path.exists():  # CPU container: build it (hipcc cross-compiles gfx950)
        import importlib.util

        spec = importlib.util.spec_from_file_location("ada_build", lib_path.parent / "build.py")
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import autoregressive_decode_attention_amd as m

    return m


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ada_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("ada_kv_append", "ada_decode_attn_gqa", "ada_decode_attn_gqa_ex",
                     "ada_decode_num_splits", "ada_decode_workspace_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol(ada):
    lib = ctypes.CDLL(str(ada.LIB_PATH))
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    assert sorted(ada.EXPORTS) == declared_functions()


def test_abi_version_and_status_strings(ada):
    assert ada.abi_version() == 3
    for code in range(-12, 1):
        assert ada.status_string(code) and ada.status_string(code) != "unknown status"
    assert ada.status_string(-99) == "unknown status"


# Fake, 16-byte aligned, never dereferenced device addresses: every call below
# must be rejected by host validation before any HIP call.
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
P3 = ctypes.c_void_p(0x30000)
P4 = ctypes.c_void_p(0x40000)
P5 = ctypes.c_void_p(0x50000)
MIS = ctypes.c_void_p(0x10008)
NUL = ctypes.c_void_p(0)


def decode(ada, q=P, k=P2, v=P3, lens=P4, B=1, Hq=32, Hkv=8, D=128, S=2048, mkl=400, scale=0.088,
           dtype=0, out=P5, ws=NUL, ws_bytes=0, splits=1):
    return ada._lib.ada_decode_attn_gqa_ex(q, k, v, lens, B, Hq, Hkv, D, S, mkl, ctypes.c_float(scale), dtype,
                                           out, ws, ws_bytes, NUL, splits)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=2), -4),
    (dict(dtype=-1), -4),
    (dict(q=NUL), -1),
    (dict(k=NUL), -1),
    (dict(v=NUL), -1),
    (dict(lens=NUL, out=NUL), -1),     # NULL lengths are the lockstep form; NULL out is not
    (dict(out=NUL), -1),
    (dict(B=-1), -2),
    (dict(Hq=0), -2),
    (dict(Hkv=0), -2),
    (dict(S=0), -2),
    (dict(Hq=30, Hkv=8), -3),
    (dict(Hq=72, Hkv=8), -3),
    (dict(D=64), -5),
    (dict(D=256), -5),
    (dict(scale=float("inf")), -6),
    (dict(scale=float("nan")), -6),
    (dict(mkl=2049), -2),
    (dict(splits=-1), -8),
    (dict(splits=257), -8),
    (dict(q=MIS), -9),
    (dict(k=MIS), -9),
    (dict(out=MIS), -9),
    (dict(splits=2), -7),
    (dict(splits=2, ws=P, ws_bytes=100), -7),
    (dict(B=0, q=NUL, k=NUL, v=NUL, lens=NUL, out=NUL), 0),
])
def test_decode_validation(ada, kwargs, status):
    assert decode(ada, **kwargs) == status


def test_workspace_too_small_by_one_byte(ada):
    need = ada.decode_workspace_bytes(1, 32, 8, 128, 3)
    assert decode(ada, splits=3, ws=P, ws_bytes=need - 1) == -7
    mis = decode(ada, splits=3, ws=MIS, ws_bytes=need)
    assert mis == -9


def test_append_validation(ada):
    f = ada._lib.ada_kv_append
    assert f(P, P2, P3, P4, P5, 1, 8, 16, 128, 5, NUL) == -4
    assert f(NUL, P2, P3, P4, P5, 1, 8, 16, 128, 0, NUL) == -1
    assert f(P, P2, P3, P4, NUL, 1, 8, 16, 128, 0, NUL) == -1
    assert f(P, P2, P3, P4, P5, -1, 8, 16, 128, 0, NUL) == -2
    assert f(P, P2, P3, P4, P5, 1, 0, 16, 128, 0, NUL) == -2
    assert f(P, P2, P3, P4, P5, 1, 8, 0, 128, 0, NUL) == -2
    assert f(P, P2, P3, P4, P5, 1, 8, 16, 64, 0, NUL) == -5
    assert f(MIS, P2, P3, P4, P5, 1, 8, 16, 128, 0, NUL) == -9
    assert f(NUL, NUL, NUL, NUL, NUL, 0, 8, 16, 128, 0, NUL) == 0
    # rows * 16 chunks must be indexable by the launch's 32-bit thread ids
    assert f(P, P2, P3, P4, P5, 65536, 2048, 16, 128, 0, NUL) == -2
    assert f(P, P2, P3, P4, P5, 2**31 - 1, 2**31 - 1, 16, 128, 0, NUL) == -2


def test_partial_and_combine_validation(ada):
    part = ada._lib.ada_decode_partial
    comb = ada._lib.ada_decode_combine
    used = ctypes.c_int(-1)
    args = lambda **kw: [kw.get("q", P), P2, P3, kw.get("lens", P4), kw.get("B", 1), 32, 8, kw.get("D", 128), 2048,
                         400, ctypes.c_float(kw.get("scale", 0.08)), kw.get("dtype", 0), kw.get("splits", 4),
                         kw.get("ws", NUL), kw.get("ws_bytes", 0), ctypes.byref(used), NUL]
    assert part(*args(dtype=3)) == -4
    assert part(*args(q=NUL)) == -1
    assert part(*args(lens=NUL)) == -7                # NULL lengths are valid (lockstep); workspace missing
    assert part(*args(D=96)) == -5
    assert part(*args(scale=float("-inf"))) == -6
    assert part(*args(splits=300)) == -8
    assert part(*args()) == -7                        # workspace required even for the partials
    assert part(*args(ws=P, ws_bytes=10)) == -7
    assert part(*args(B=0, q=NUL, lens=NUL)) == 0 and used.value == 0
    need = ada.decode_workspace_bytes(1, 32, 8, 128, 4)
    assert comb(P, need, 1, 32, 8, 128, 0, 0, P5, NUL) == -8
    assert comb(P, need, 1, 32, 8, 128, 257, 0, P5, NUL) == -8
    assert comb(P, need - 1, 1, 32, 8, 128, 4, 0, P5, NUL) == -7
    assert comb(NUL, need, 1, 32, 8, 128, 4, 0, P5, NUL) == -7
    assert comb(P, need, 1, 32, 8, 128, 4, 0, NUL, NUL) == -1
    assert comb(P, need, 1, 32, 8, 128, 4, 0, MIS, NUL) == -9
    assert comb(P, need, 1, 30, 8, 128, 4, 0, P5, NUL) == -3
    assert comb(P, need, 1, 32, 8, 64, 4, 0, P5, NUL) == -5
    assert comb(P, need, 1, 32, 8, 128, 4, 7, P5, NUL) == -4
    assert comb(NUL, 0, 0, 32, 8, 128, 4, 0, NUL, NUL) == 0


def test_decode_step_validation(ada):
    f = ada._lib.ada_decode_step
    args = lambda **kw: [kw.get("q", P), kw.get("kn", P2), kw.get("vn", P3), P4, P5, NUL, 1, 32, 8,
                         kw.get("D", 128), 2048, kw.get("mp", 399), ctypes.c_float(0.08), kw.get("dtype", 0),
                         kw.get("out", P), kw.get("ws", NUL), kw.get("ws_bytes", 0), NUL, kw.get("splits", 2)]
    assert f(*args(mp=2048)) == -2
    assert f(*args(mp=-1)) == -2
    assert f(*args(dtype=9)) == -4
    assert f(*args(kn=NUL)) == -1
    assert f(*args(vn=NUL)) == -1
    assert f(*args(out=NUL)) == -1
    assert f(*args(q=NUL)) == -1
    assert f(*args(kn=MIS)) == -9
    assert f(*args(D=64)) == -5
    assert f(*args()) == -7                     # two splits need a workspace
    assert f(*args(splits=300)) == -8


def test_prefill_rows_per_workgroup_rule(ada):
    """Two 16-row blocks per wavefront (128 rows per workgroup) only when the
    launch keeps at least 2 workgroups per compute unit."""
    f = ada.prefill_rows_per_workgroup
    assert f(1, 32, 8, 2048, 256) == 128       # 64 row tiles x 8 units = 512 = 2 x 256
    assert f(1, 32, 8, 2017, 256) == 128       # 8068 rows: still 64 tiles
    assert f(1, 32, 8, 2016, 256) == 64        # 8064 rows: 63 x 8 = 504
    assert f(1, 32, 8, 4096, 256) == 128
    assert f(1, 32, 8, 1024, 256) == 64
    assert f(1, 32, 8, 234, 256) == 64
    assert f(1, 16, 16, 4096, 256) == 128      # MHA: 32 x 16 = 512
    assert f(1, 16, 16, 2048, 256) == 64
    assert f(16, 32, 8, 256, 256) == 128       # 8 x 128 units
    assert f(1, 32, 8, 2048, 512) == 64        # a larger device needs more work
    for bad in ((0, 32, 8, 64, 256), (1, 0, 8, 64, 256), (1, 32, 0, 64, 256), (1, 32, 8, 0, 256),
                (1, 32, 8, 64, 0), (1, 30, 8, 64, 256)):
        assert f(*bad) == 64


def test_step_graph_validation(ada):
    """Host checks of the graph-captured step: every call here is rejected
    before any HIP call, and the handle is left NULL."""
    create = ada._lib.ada_step_graph_create
    layer = lambda **kw: ada.StepLayer(*(kw.get(n, d) for n, d in (
        ("q", 0x10000), ("k_new", 0x20000), ("v_new", 0x30000), ("k_cache", 0x40000), ("v_cache", 0x50000),
        ("out", 0x60000), ("cos", None), ("sin", None))))

    def call(layers=None, n=None, pos=P, B=1, D=128, S=2048, mp=399, dtype=0, scale=0.08, handle=True):
        layers = layers if layers is not None else [layer(), layer()]
        arr = (ada.StepLayer * max(len(layers), 1))(*layers)
        h = ctypes.c_void_p(0xdead)
        rc = create(arr, len(layers) if n is None else n, pos, B, 32, 8, D, S, mp, ctypes.c_float(scale), dtype, 1,
                    NUL, 0, ctypes.byref(h) if handle else None)
        if handle:
            assert h.value is None, "the handle must be NULL after an error"
        return rc

    assert call(handle=False) == -1
    assert call(n=0) == -2
    assert call(pos=NUL) == -1
    assert call(pos=ctypes.c_void_p(0x10002)) == -9
    assert call(mp=2048) == -2
    assert call(mp=-1) == -2
    assert call(dtype=5) == -4
    assert call(D=64) == -5
    assert call(scale=float("inf")) == -6
    assert call(layers=[layer(), layer(q=None)]) == -1          # the second layer is checked too
    assert call(layers=[layer(k_cache=0x40008)]) == -9
    assert create(None, 1, P, 1, 32, 8, 128, 2048, 399, ctypes.c_float(0.08), 0, 1, NUL, 0,
                  ctypes.byref(ctypes.c_void_p())) == -1
    assert ada._lib.ada_step_graph_launch(None, NUL) == -1
    ada._lib.ada_step_graph_destroy(None)  # a no-op


def test_rope_kv_append_validation(ada):
    f = ada._lib.ada_rope_kv_append
    # q, q_out, k_new, v_new, cos, sin, k_cache, v_cache, pos, B, Hq, Hkv, S, D, dtype, stream
    args = lambda **kw: [kw.get("q", P), kw.get("qo", P2), kw.get("kn", P3), kw.get("vn", P4), kw.get("cos", P5),
                         kw.get("sin", P), kw.get("kc", P2), kw.get("vc", P3), kw.get("pos", P4), kw.get("B", 1),
                         kw.get("Hq", 32), 8, 16, kw.get("D", 128), kw.get("dtype", 0), NUL]
    assert f(*args(dtype=3)) == -4
    assert f(*args(D=64)) == -5
    assert f(*args(B=-1)) == -2
    assert f(*args(Hq=0)) == -2                  # a query needs heads
    assert f(*args(qo=NUL)) == -1                # q without q_out
    assert f(*args(q=NUL)) == -1                 # q_out without q
    assert f(*args(cos=NUL)) == -1
    assert f(*args(sin=NUL)) == -1
    assert f(*args(pos=NUL)) == -1
    assert f(*args(cos=MIS)) == -9
    assert f(*args(qo=MIS)) == -9
    assert f(*args(B=0, q=NUL, qo=NUL, kn=NUL, vn=NUL, cos=NUL, sin=NUL, kc=NUL, vc=NUL, pos=NUL)) == 0


def test_decode_step_rope_validation(ada):
    f = ada._lib.ada_decode_step_rope
    args = lambda **kw: [kw.get("q", P), kw.get("kn", P2), kw.get("vn", P3), kw.get("cos", P4), kw.get("sin", P5),
                         P, P2, NUL, 1, 32, 8, kw.get("D", 128), 2048, kw.get("mp", 399), ctypes.c_float(0.08),
                         kw.get("dtype", 0), kw.get("out", P3), kw.get("ws", NUL), kw.get("ws_bytes", 0), NUL,
                         kw.get("splits", 2)]
    assert f(*args(cos=NUL)) == -1
    assert f(*args(sin=NUL)) == -1
    assert f(*args(cos=MIS)) == -9
    assert f(*args(sin=MIS)) == -9
    assert f(*args(dtype=7)) == -4
    assert f(*args(mp=2048)) == -2
    assert f(*args(D=64)) == -5
    assert f(*args(kn=NUL)) == -1
    assert f(*args()) == -7                      # two splits need a workspace
    assert f(*args(splits=300)) == -8


def test_prefill_validation(ada):
    f = ada._lib.ada_prefill_attn_gqa
    # q, k, v, start, B, Hq, Hkv, T, D, S, scale, dtype, out, stream
    args = lambda **kw: [kw.get("q", P), kw.get("k", P2), kw.get("v", P3), NUL, kw.get("B", 1), kw.get("Hq", 32),
                         kw.get("Hkv", 8), kw.get("T", 16), kw.get("D", 128), kw.get("S", 64),
                         ctypes.c_float(kw.get("scale", 0.08)),
                         kw.get("dtype", 0), kw.get("out", P4), NUL]
    assert f(*args(dtype=2)) == -4
    assert f(*args(Hq=12)) == -3
    assert f(*args(Hq=72)) == -3              # group 9
    assert f(*args(D=64)) == -5
    assert f(*args(T=-1)) == -2
    assert f(*args(scale=float("inf"))) == -6
    assert f(*args(q=NUL)) == -1
    assert f(*args(out=NUL)) == -1
    assert f(*args(q=MIS)) == -9
    assert f(*args(T=0, q=NUL, k=NUL, v=NUL, out=NUL)) == 0
    assert f(*args(S=1 << 23)) == -2          # a KV head's slab must stay under 2 GiB (32-bit offsets)
    assert f(*args(S=1 << 23, T=0)) == -2
    g = ada._lib.ada_prefill_append
    gargs = lambda **kw: [kw.get("kn", P), P2, P3, P4, NUL, kw.get("B", 1), 8, kw.get("T", 16), 64, kw.get("D", 128),
                          kw.get("dtype", 1), NUL]
    assert g(*gargs(dtype=5)) == -4
    assert g(*gargs(D=96)) == -5
    assert g(*gargs(T=-3)) == -2
    assert g(*gargs(kn=NUL)) == -1
    assert g(*gargs(kn=MIS)) == -9
    assert g(*gargs(T=0, kn=NUL)) == 0


def test_workspace_bytes_arithmetic(ada):
    r256 = lambda x: (x + 255) // 256 * 256
    for B, Hq, Hkv, splits in ((1, 32, 8, 4), (8, 32, 8, 8), (4, 32, 8, 33), (1, 16, 16, 32), (3, 6, 3, 7)):
        rows = B * Hq * splits
        want = r256(rows * 8) + r256(rows * 128 * 4)
        assert ada.decode_workspace_bytes(B, Hq, Hkv, 128, splits) == want
    assert ada.decode_workspace_bytes(8, 32, 8, 128, 1) == r256(8 * 32 * 8) + r256(8 * 32 * 512)
    assert ada.decode_workspace_bytes(8, 32, 8, 128, 0) == 0
    assert ada.decode_workspace_bytes(0, 32, 8, 128, 4) == 0
    # sizes no call can use report 0 instead of wrapping
    assert ada.decode_workspace_bytes(2**31 - 1, 2**31 - 1, 1, 128, 256) == 0
    assert ada.decode_workspace_bytes(65535, 8 * 65535, 65535, 128, 256) == r256(65535 * 8 * 65535 * 256 * 8) + \
        r256(65535 * 8 * 65535 * 256 * 512)


def test_split_heuristic_properties(ada):
    ns = ada.decode_num_splits
    # worked examples on a 256-CU device (the values the tuning sweeps favoured)
    assert ns(8, 32, 8, 32768, 256) == 4     # long context: one workgroup per CU, 8192-slot splits
    assert ns(1, 16, 16, 4096, 256) == 16    # MHA kv 4096: one workgroup per CU, 256-slot splits
    assert ns(1, 16, 16, 8192, 256) == 16
    assert ns(8, 32, 8, 65536, 256) == 8     # 16384-slot splits would exceed 8192 -> doubled
    assert ns(1, 16, 16, 1024, 256) == 16    # capped by 64-slot splits
    assert ns(4, 32, 8, 8192, 256) == 8      # MiniCPM shape: one workgroup per CU
    assert ns(1, 32, 8, 400, 256) == 7       # tiny
    assert ns(1, 32, 8, 235, 256) == 1       # at most 256 slots: one split, no combine launch
    assert ns(1, 16, 16, 256, 256) == 1
    assert ns(1, 16, 16, 257, 256) == 5
    for B in (1, 2, 4, 8, 16, 64):
        for Hq, Hkv in ((16, 16), (32, 8), (8, 1)):
            for n in (1, 63, 64, 65, 400, 1258, 4096, 8191, 32768, 131072, 1 << 20):
                s = ns(B, Hq, Hkv, n, 256)
                assert 1 <= s <= 256
                chunk = -(-n // s)
                chunk = -(-chunk // 64) * 64
                # the count is the one the 64-slot rounding yields, and every split is live
                assert s == -(-n // chunk)
                assert s <= max(1, -(-n // 64))
                # splits longer than 8192 slots only when the split count is at its cap
                if chunk > 8192 + 63:
                    assert s * 2 > -(-n // 64) or s * 2 > 256
                # splitting never asks for more than one workgroup per CU unless rows are long
                if s > 1 and B * Hkv * s > 256:
                    assert chunk > 4096 - 64
    assert ns(0, 8, 8, 100, 256) == 1
    assert ns(1, 8, 8, 0, 256) == 1
    assert ns(1, 8, 8, 100, 0) == 1


def test_decode_plan_export(ada):
    """ada_decode_plan: the heuristic's count (as ada_decode_num_splits) with
    a chunk that covers the prefix in whole 64-slot tiles, or a forced count's
    near-equal ranges; the binding sizes workspaces with it."""
    plan = lambda B, Hq, Hkv, n, sp, cus=256: ada.decode_plan(B, Hq, Hkv, n, sp, cus)
    for B, Hq, Hkv in ((1, 32, 8), (8, 32, 8), (1, 16, 16), (4, 32, 8), (3, 12, 3)):
        for n in (1, 64, 65, 235, 400, 1258, 4096, 8192, 32768, 1 << 22):
            s, c = plan(B, Hq, Hkv, n, 0)
            assert s == ada.decode_num_splits(B, Hq, Hkv, n, 256)
            assert s * c >= n > (s - 1) * c
            if n > 256:
                assert c % 64 == 0
            for forced in (1, 2, 3, 7, 40, 256):
                s, c = plan(B, Hq, Hkv, n, forced)
                assert c == -(-n // forced) and s == -(-n // c) and s <= forced
    assert plan(8, 32, 8, 32768, 0) == (4, 8192)
    assert plan(1, 16, 16, 4096, 0) == (16, 256)
    assert plan(1, 32, 8, 0, 5) == (1, 1)
    f = ada._lib.ada_decode_plan
    one = ctypes.c_int(0)
    assert f(1, 32, 8, 100, 0, 256, None, ctypes.byref(one)) == -1
    assert f(1, 32, 8, 100, 0, 256, ctypes.byref(one), None) == -1
    assert f(1, 32, 8, 100, -1, 256, ctypes.byref(one), ctypes.byref(one)) == -8
    assert f(1, 32, 8, 100, 257, 256, ctypes.byref(one), ctypes.byref(one)) == -8


def test_hbm_read_validation(ada):
    f = ada._lib.ada_hbm_read
    assert f(P, 1 << 20, P2, 0, NUL) == -2          # no workgroup
    assert f(P, 1 << 20, P2, (1 << 20) + 1, NUL) == -2
    assert f(P, (1 << 20) + 8, P2, 256, NUL) == -2  # not whole 16-byte chunks
    assert f(NUL, 1 << 20, P2, 256, NUL) == -1
    assert f(P, 1 << 20, NUL, 256, NUL) == -1
    assert f(MIS, 1 << 20, P2, 256, NUL) == -9
    assert f(P, 1 << 20, ctypes.c_void_p(0x20002), 256, NUL) == -9
    assert f(NUL, 0, NUL, 256, NUL) == 0           # nothing to read


def test_noalloc_validation(ada):
    """ada_decode_attn_gqa_noalloc: the decode checks, then the limit of the
    static scratch (forced split counts need no device, so this runs on the
    CPU); a call over the limit is rejected before any HIP call."""
    f = ada._lib.ada_decode_attn_gqa_noalloc
    sc = ctypes.c_float(0.088)

    def call(B=1, Hq=32, Hkv=8, D=128, S=4096, n=4096, dtype=1, out=P4, splits=8, q=P):
        return f(q, P2, P3, NUL, B, Hq, Hkv, D, S, n, sc, dtype, out, NUL, splits)

    assert call(dtype=7) == -4
    assert call(D=64) == -5
    assert call(Hq=36) == -3
    assert call(out=NUL) == -1
    assert call(q=NUL) == -1
    assert call(out=MIS) == -9
    assert call(splits=300) == -8
    assert call(n=5000) == -2
    assert call(B=0, q=NUL, out=NUL) == 0
    limit = 4 << 20
    # 64 rows x 64 heads x 256 splits of partials: far beyond the scratch
    assert ada.decode_workspace_bytes(64, 64, 8, 128, 256) > limit
    assert call(B=64, Hq=64, S=1 << 16, n=1 << 16, splits=256) == -12
    # the largest forced count that fits for batch 8 x 32 heads (the long-context shape) is checked exactly
    fits = max(s for s in range(1, 257) if ada.decode_workspace_bytes(8, 32, 8, 128, s) <= limit)
    assert ada.decode_workspace_bytes(8, 32, 8, 128, fits + 1) > limit
    assert call(B=8, S=32768, n=32768, splits=fits + 1) == -12
    assert ada.status_string(-12) != "unknown status"
