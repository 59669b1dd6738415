"""CPU oracle for single-token decode attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. It wraps ``liboracle.so``, built from ``ada_oracle.c`` with the
host C compiler, through ctypes. It shares no code with the GPU library and
imports nothing from it.

The rotary map applied to the new token's query and key before the cache
write lives in ``rope.py`` (plain Python, exact rationals); ``decode_step_rope``
below composes it with the append and the decode in the page's order.

The C source states the definition it computes and the page sections it
follows. Every function is pinned by ``tests/test_oracle_pins.py`` to results
obtained another way (an independent library attention routine, closed forms,
invariants, exhaustive decoder checks), and ``tests/test_oracle_mutants.py``
shows that plausible mistakes in the source fail those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from pathlib import Path

import numpy as np

ORACLE_DIR = Path(__file__).resolve().parent
SOURCE = ORACLE_DIR / "ada_oracle.c"
LIBRARY = ORACLE_DIR / "liboracle.so"

DTYPES = {"fp16": 0, "bf16": 1}


def build(source: Path | str = SOURCE, output: Path | str = LIBRARY, openmp: bool = True) -> Path:
    """Compile the oracle into a shared library with the host C compiler."""
    output = Path(output)
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra"]
    if openmp:
        cmd.append("-fopenmp")
    cmd += ["-o", str(output) + ".tmp", str(source), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(str(output) + ".tmp", output)
    return output


def build_from_text(text: str, directory: str | None = None) -> Path:
    """Compile oracle source given as text (used by the mutation tests)."""
    d = Path(directory or tempfile.mkdtemp(prefix="ada_oracle_"))
    src = d / "ada_oracle_variant.c"
    src.write_text(text)
    return build(src, d / "liboracle_variant.so", openmp=False)


def _bits(x) -> np.ndarray:
    """Raw 16-bit patterns of a torch fp16/bf16 tensor or a uint16 array."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy inputs must hold raw uint16 bit patterns")
        return np.ascontiguousarray(x)
    import torch

    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"expected a 16-bit float tensor, got {x.dtype}")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _dtype_name(x, dtype: str | None) -> str:
    if dtype is not None:
        return dtype
    import torch

    return {torch.float16: "fp16", torch.bfloat16: "bf16"}[x.dtype]


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: Path | str = LIBRARY):
        self.path = Path(path)
        lib = ctypes.CDLL(str(self.path))
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        c_int = ctypes.c_int
        lib.ada_oracle_decode.argtypes = [u16p, u16p, u16p, i32p, c_int, c_int, c_int, c_int, c_int,
                                          ctypes.c_double, c_int, f64p]
        lib.ada_oracle_decode.restype = c_int
        lib.ada_oracle_kv_append.argtypes = [u16p, u16p, u16p, u16p, i32p, c_int, c_int, c_int, c_int]
        lib.ada_oracle_kv_append.restype = c_int
        lib.ada_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.ada_oracle_f16_to_f64.restype = ctypes.c_double
        lib.ada_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.ada_oracle_bf16_to_f64.restype = ctypes.c_double
        lib.ada_oracle_prefill.argtypes = [u16p, u16p, u16p, i32p, c_int, c_int, c_int, c_int, c_int, c_int,
                                           ctypes.c_double, c_int, f64p]
        lib.ada_oracle_prefill.restype = c_int
        lib.ada_oracle_prefill_append.argtypes = [u16p, u16p, u16p, u16p, i32p, c_int, c_int, c_int, c_int, c_int]
        lib.ada_oracle_prefill_append.restype = c_int
        lib.ada_oracle_threads.argtypes = []
        lib.ada_oracle_threads.restype = c_int
        lib.ada_oracle_set_threads.argtypes = [c_int]
        lib.ada_oracle_set_threads.restype = None
        self._lib = lib

    def threads(self) -> int:
        return int(self._lib.ada_oracle_threads())

    def set_threads(self, n: int) -> None:
        """Threads later calls may use (the results do not depend on it)."""
        self._lib.ada_oracle_set_threads(int(n))

    def decode_bits(self, bits: np.ndarray, dtype: str) -> np.ndarray:
        """Decode an array of raw 16-bit patterns to float64, one by one."""
        fn = self._lib.ada_oracle_bf16_to_f64 if dtype == "bf16" else self._lib.ada_oracle_f16_to_f64
        flat = np.asarray(bits, dtype=np.uint16).ravel()
        return np.array([fn(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))

    def decode(self, q, k_cache, v_cache, kv_len, scale: float, dtype: str | None = None) -> np.ndarray:
        """out[b, h, :] in float64 for q [B, Hq, D], caches [B, Hkv, S, D]."""
        dt = _dtype_name(q, dtype)
        qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
        if qb.ndim == 4:  # [B, Hq, 1, D]
            qb = qb.reshape(qb.shape[0], qb.shape[1], qb.shape[3])
        batch, n_head, head_dim = qb.shape
        kb_, n_kv_head, capacity, kd = kb.shape
        if kb.shape != vb.shape or kb_ != batch or kd != head_dim:
            raise ValueError("inconsistent shapes")
        lens = np.ascontiguousarray(np.asarray(
            kv_len.cpu().numpy() if hasattr(kv_len, "cpu") else kv_len, dtype=np.int32).reshape(batch))
        out = np.zeros((batch, n_head, head_dim), dtype=np.float64)
        rc = self._lib.ada_oracle_decode(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                         _ptr(vb, ctypes.c_uint16), _ptr(lens, ctypes.c_int32),
                                         batch, n_head, n_kv_head, head_dim, capacity,
                                         float(scale), DTYPES[dt], _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError(f"oracle decode failed with status {rc}")
        return out

    def prefill(self, q, k_cache, v_cache, start, scale: float, dtype: str | None = None) -> np.ndarray:
        """Causal prefill: out[b, h, t, :] in float64 for q [B, Hq, T, D], caches
        [B, Hkv, S, D]; token t of row b attends slots 0 .. start[b] + t."""
        dt = _dtype_name(q, dtype)
        qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
        batch, n_head, q_len, head_dim = qb.shape
        kb_, n_kv_head, capacity, kd = kb.shape
        if kb.shape != vb.shape or kb_ != batch or kd != head_dim:
            raise ValueError("inconsistent shapes")
        st = np.ascontiguousarray(np.asarray(
            start.cpu().numpy() if hasattr(start, "cpu") else start, dtype=np.int32).reshape(batch))
        out = np.zeros((batch, n_head, q_len, head_dim), dtype=np.float64)
        rc = self._lib.ada_oracle_prefill(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                          _ptr(vb, ctypes.c_uint16), _ptr(st, ctypes.c_int32), batch, n_head,
                                          n_kv_head, q_len, head_dim, capacity, float(scale), DTYPES[dt],
                                          _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError(f"oracle prefill failed with status {rc}")
        return out

    def prefill_append(self, k_new, v_new, k_cache, v_cache, start):
        """Return updated copies of the caches with the T new rows [B, Hkv, T, D]
        written at slots start[b] .. start[b] + T - 1 (inputs not modified)."""
        kn, vn = np.ascontiguousarray(_bits(k_new)), np.ascontiguousarray(_bits(v_new))
        kc, vc = _bits(k_cache).copy(), _bits(v_cache).copy()
        batch, n_kv_head, capacity, head_dim = kc.shape
        q_len = kn.shape[2]
        if kn.shape != (batch, n_kv_head, q_len, head_dim) or vn.shape != kn.shape:
            raise ValueError("k_new / v_new must be [B, Hkv, T, D]")
        st = np.ascontiguousarray(np.asarray(
            start.cpu().numpy() if hasattr(start, "cpu") else start, dtype=np.int32).reshape(batch))
        rc = self._lib.ada_oracle_prefill_append(_ptr(kn, ctypes.c_uint16), _ptr(vn, ctypes.c_uint16),
                                                 _ptr(kc, ctypes.c_uint16), _ptr(vc, ctypes.c_uint16),
                                                 _ptr(st, ctypes.c_int32), batch, n_kv_head, q_len, capacity,
                                                 head_dim)
        if rc != 0:
            raise ValueError(f"oracle prefill_append failed with status {rc}")
        return kc, vc

    def kv_append(self, k_new, v_new, k_cache, v_cache, pos):
        """Return updated copies of the caches (inputs are not modified)."""
        kn, vn = _bits(k_new), _bits(v_new)
        kc, vc = _bits(k_cache).copy(), _bits(v_cache).copy()
        batch, n_kv_head, capacity, head_dim = kc.shape
        p = np.ascontiguousarray(np.asarray(
            pos.cpu().numpy() if hasattr(pos, "cpu") else pos, dtype=np.int32).reshape(batch))
        kn = np.ascontiguousarray(kn.reshape(batch, n_kv_head, head_dim))
        vn = np.ascontiguousarray(vn.reshape(batch, n_kv_head, head_dim))
        rc = self._lib.ada_oracle_kv_append(_ptr(kn, ctypes.c_uint16), _ptr(vn, ctypes.c_uint16),
                                            _ptr(kc, ctypes.c_uint16), _ptr(vc, ctypes.c_uint16),
                                            _ptr(p, ctypes.c_int32), batch, n_kv_head, capacity, head_dim)
        if rc != 0:
            raise ValueError(f"oracle kv_append failed with status {rc}")
        return kc, vc


def decode_step_rope(ora: "Oracle", q, k_new, v_new, cos, sin, k_cache, v_cache, pos, scale: float,
                     dtype: str | None = None):
    """One decode step with rotary embedding, in the order of the MiniCPM4
    forward_step ("VoxCPM #395", section 4): rotate the new query and key
    (``rope.rope``), write the rotated key and the value at slot pos[b] of
    every KV head, then attend over slots [0, pos[b]] (kv_len = pos[b] + 1,
    clamped to the capacity by the decode; a position outside the cache
    writes nothing).

    q [B, Hq, D], k_new / v_new [B, Hkv, D], cos / sin [B, D], caches
    [B, Hkv, S, D] (16-bit tensors or uint16 patterns). Returns (out float64
    [B, Hq, D], q_rot bits, k_cache bits, v_cache bits); the inputs are not
    modified.
    """
    from . import rope as _rope

    dt = _dtype_name(q, dtype)
    qb = _bits(q)
    if qb.ndim == 4:
        qb = qb.reshape(qb.shape[0], qb.shape[1], qb.shape[3])
    batch = qb.shape[0]
    kn = _bits(k_new).reshape(batch, -1, qb.shape[-1])
    q_rot = _rope.rope(qb, _bits(cos), _bits(sin), dt)
    k_rot = _rope.rope(kn, _bits(cos), _bits(sin), dt)
    kc, vc = ora.kv_append(k_rot, _bits(v_new), _bits(k_cache), _bits(v_cache), pos)
    p = np.asarray(pos.cpu().numpy() if hasattr(pos, "cpu") else pos, dtype=np.int64).reshape(batch)
    lens = np.clip(p + 1, 0, None).astype(np.int32)
    out = ora.decode(q_rot, kc, vc, lens, scale, dt)
    return out, q_rot, kc, vc


_DEFAULT: Oracle | None = None


def load() -> Oracle:
    """The oracle built from ``ada_oracle.c``; compiled here if not yet built."""
    global _DEFAULT
    if _DEFAULT is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
