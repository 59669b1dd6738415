"""Single-token decode attention for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libada.so``, whose C ABI is declared in
``include/ada.h``. Every step of the computation runs in the library's HIP
kernels; this module only checks tensors, takes their device pointers and the
current HIP stream, and manages a cached split workspace. PyTorch is used for
device memory and streams only.

The functions keep the C names without the ``ada_`` prefix:

* ``kv_append(k_new, v_new, k_cache, v_cache, pos)``
* ``decode_attn_gqa(q, k_cache, v_cache, kv_len, scale=None, out=None, max_kv_len=None)``
* ``decode_attn_gqa_ex(..., num_splits=...)``
* ``decode_attn_gqa_noalloc(...)``: the same with the library's static scratch (no allocation)
* ``decode_step(q, k_new, v_new, k_cache, v_cache, pos, ...)``: append + decode in one call
* ``decode_step_rope(q, k_new, v_new, cos, sin, k_cache, v_cache, pos, ...)`` and
  ``rope_kv_append(q, k_new, v_new, cos, sin, k_cache, v_cache, pos)``: the same
  with the rotary embedding of the new query and key
* ``step_graph(layers, pos, max_pos, ...)``: every layer's decode step plus the
  position advance recorded once as a HIP graph (``StepGraph.launch()``)
* ``decode_partial(q, k_cache, v_cache, kv_len, ...)`` and
  ``decode_combine(workspace, num_splits, out, n_kv_head)``: the two halves
* ``prefill_append(k_new, v_new, k_cache, v_cache, start)`` and
  ``prefill_attn_gqa(q, k_cache, v_cache, start, ...)``: prompt prefill
* ``decode_num_splits``, ``decode_plan``, ``decode_workspace_bytes``, ``prefill_rows_per_workgroup``,
  ``device_num_cus``, ``status_string``, ``last_hip_error``, ``abi_version``.
* ``hbm_read(src, sink, workgroups)``: measurement only, a plain streaming read

There is no fallback: if the library is missing, importing this package
raises ImportError.
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path

import torch  # loads the HIP runtime the library then shares

PKG_DIR = Path(__file__).resolve().parent
LIB_PATH = PKG_DIR / "libada.so"

F16, BF16 = 0, 1
_DTYPE_CODES = {torch.float16: F16, torch.bfloat16: BF16}
HEAD_DIM = 128
MAX_SPLITS = 256

STATUS = {
    0: "ADA_OK", -1: "ADA_ERR_NULL", -2: "ADA_ERR_SHAPE", -3: "ADA_ERR_GQA", -4: "ADA_ERR_DTYPE",
    -5: "ADA_ERR_HEAD_DIM", -6: "ADA_ERR_SCALE", -7: "ADA_ERR_WORKSPACE", -8: "ADA_ERR_SPLITS",
    -9: "ADA_ERR_ALIGN", -10: "ADA_ERR_HIP", -11: "ADA_ERR_DEVICE", -12: "ADA_ERR_SCRATCH",
}

EXPORTS = (
    "ada_abi_version", "ada_status_string", "ada_last_hip_error", "ada_device_num_cus",
    "ada_kv_append", "ada_decode_num_splits", "ada_decode_plan", "ada_decode_workspace_bytes",
    "ada_decode_attn_gqa", "ada_decode_attn_gqa_ex", "ada_decode_partial", "ada_decode_combine",
    "ada_decode_step", "ada_rope_kv_append", "ada_decode_step_rope", "ada_prefill_append",
    "ada_prefill_attn_gqa", "ada_prefill_rows_per_workgroup", "ada_step_graph_create", "ada_step_graph_launch", "ada_step_graph_destroy",
    "ada_hbm_read", "ada_decode_attn_gqa_noalloc",
)


class StepLayer(ctypes.Structure):
    """``ada_step_layer``: the buffers of one layer of a graph-captured step."""
    _fields_ = [(name, ctypes.c_void_p) for name in ("q", "k_new", "v_new", "k_cache", "v_cache", "out", "cos", "sin")]


class AdaError(RuntimeError):
    """A libada call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({_status_text(status)})"
        if status == -10:
            msg += f", hipError {last_hip_error()}"
        super().__init__(msg)


def _declare(lib):
    c_int, c_void_p, c_size_t, c_float = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    decode_args = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                   c_float, c_int, c_void_p, c_void_p, c_size_t, c_void_p]
    sigs = {
        "ada_abi_version": ([], c_int),
        "ada_status_string": ([c_int], ctypes.c_char_p),
        "ada_last_hip_error": ([], c_int),
        "ada_device_num_cus": ([c_int, ctypes.POINTER(c_int)], c_int),
        "ada_kv_append": ([c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                           c_int, c_void_p], c_int),
        "ada_decode_num_splits": ([c_int, c_int, c_int, c_int, c_int], c_int),
        "ada_decode_plan": ([c_int] * 6 + [ctypes.POINTER(c_int), ctypes.POINTER(c_int)], c_int),
        "ada_decode_workspace_bytes": ([c_int, c_int, c_int, c_int, c_int], c_size_t),
        "ada_decode_attn_gqa": (decode_args, c_int),
        "ada_decode_attn_gqa_ex": (decode_args + [c_int], c_int),
        "ada_decode_attn_gqa_noalloc": ([c_void_p] * 4 + [c_int] * 6 + [c_float, c_int, c_void_p, c_void_p, c_int],
                                        c_int),
        "ada_decode_partial": ([c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                c_float, c_int, c_int, c_void_p, c_size_t, ctypes.POINTER(c_int), c_void_p], c_int),
        "ada_decode_combine": ([c_void_p, c_size_t, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p],
                               c_int),
        "ada_decode_step": ([c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                             c_int, c_int, c_float, c_int, c_void_p, c_void_p, c_size_t, c_void_p, c_int], c_int),
        "ada_rope_kv_append": ([c_void_p] * 9 + [c_int] * 6 + [c_void_p], c_int),
        "ada_prefill_append": ([c_void_p] * 5 + [c_int] * 6 + [c_void_p], c_int),
        "ada_prefill_attn_gqa": ([c_void_p] * 4 + [c_int] * 6 + [c_float, c_int, c_void_p, c_void_p], c_int),
        "ada_decode_step_rope": ([c_void_p] * 8 + [c_int] * 6 + [c_float, c_int, c_void_p, c_void_p, c_size_t,
                                                                 c_void_p, c_int], c_int),
        "ada_step_graph_create": ([ctypes.POINTER(StepLayer), c_int, c_void_p] + [c_int] * 6 +
                                  [c_float, c_int, c_int, c_void_p, c_size_t, ctypes.POINTER(c_void_p)], c_int),
        "ada_step_graph_launch": ([c_void_p, c_void_p], c_int),
        "ada_prefill_rows_per_workgroup": ([c_int] * 5, c_int),
        "ada_step_graph_destroy": ([c_void_p], None),
        "ada_hbm_read": ([c_void_p, c_size_t, c_void_p, c_int, c_void_p], c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def load_library(path: Path | str = LIB_PATH):
    """Load a build of libada and declare its C signatures."""
    path = Path(path)
    if not path.exists():
        raise ImportError(f"{path} is not built; run `python autoregressive_decode_attention_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    return _declare(ctypes.CDLL(str(path)))


_lib = load_library()


def _status_text(status: int) -> str:
    return _lib.ada_status_string(int(status)).decode()


def status_string(status: int) -> str:
    return _status_text(status)


def last_hip_error() -> int:
    return int(_lib.ada_last_hip_error())


def abi_version() -> int:
    return int(_lib.ada_abi_version())


def _check(status: int, where: str):
    if status != 0:
        raise AdaError(status, where)


def device_num_cus(device=None) -> int:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    n = ctypes.c_int(0)
    _check(_lib.ada_device_num_cus(dev.index if dev.index is not None else torch.cuda.current_device(),
                                   ctypes.byref(n)), "ada_device_num_cus")
    return n.value


_CUS: dict = {}


def _cus(device: torch.device) -> int:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _CUS:
        _CUS[idx] = device_num_cus(torch.device("cuda", idx))
    return _CUS[idx]


def decode_num_splits(batch: int, n_head: int, n_kv_head: int, max_kv_len: int, num_cus: int | None = None) -> int:
    if num_cus is None:
        num_cus = _cus(torch.device("cuda", torch.cuda.current_device()))
    return int(_lib.ada_decode_num_splits(int(batch), int(n_head), int(n_kv_head), int(max_kv_len), int(num_cus)))


def decode_plan(batch: int, n_head: int, n_kv_head: int, max_kv_len: int, num_splits: int = 0,
                num_cus: int | None = None) -> tuple:
    """(splits, chunk) of a decode call over ``max_kv_len`` slots, from the
    library (``ada_decode_plan``): the heuristic on ``num_cus`` compute units
    (default: the current device) when ``num_splits`` is 0, else the forced
    count's near-equal ranges."""
    if num_splits == 0 and num_cus is None:
        num_cus = _cus(torch.device("cuda", torch.cuda.current_device()))
    splits, chunk = ctypes.c_int(0), ctypes.c_int(0)
    _check(_lib.ada_decode_plan(int(batch), int(n_head), int(n_kv_head), int(max_kv_len), int(num_splits),
                                int(num_cus or 0), ctypes.byref(splits), ctypes.byref(chunk)), "ada_decode_plan")
    return splits.value, chunk.value


def prefill_rows_per_workgroup(batch: int, n_head: int, n_kv_head: int, q_len: int, num_cus: int | None = None) -> int:
    """Query rows per workgroup prefill_attn_gqa uses (64 or 128) on a device
    with ``num_cus`` compute units (default: the current device)."""
    cus = device_num_cus() if num_cus is None else int(num_cus)
    return int(_lib.ada_prefill_rows_per_workgroup(int(batch), int(n_head), int(n_kv_head), int(q_len), cus))


def decode_workspace_bytes(batch: int, n_head: int, n_kv_head: int, head_dim: int, num_splits: int) -> int:
    return int(_lib.ada_decode_workspace_bytes(int(batch), int(n_head), int(n_kv_head), int(head_dim),
                                               int(num_splits)))


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of ``nbytes`` bytes on ``device`` (scratch; needs no preparation)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# Cached workspaces, one per (device, stream): calls on one stream are ordered.
_WORKSPACES: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    key = (device.index, _stream(device))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(max(nbytes, 2 * (ws.numel() if ws is not None else 0)), device)
        _WORKSPACES[key] = ws
    return ws


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              pos) -> None:
    """Write k_new/v_new [B, Hkv, D] (or [B, Hkv, 1, D]) into slot pos[b] of the
    caches [B, Hkv, S, D], in place, on the current stream. ``pos``: int32
    device tensor [B], or host ints (copied to the device)."""
    _require(k_cache.is_cuda and k_cache.dim() == 4, "k_cache must be a 4-d GPU tensor [B, Hkv, S, D]")
    B, Hkv, S, D = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "v_cache shape must equal k_cache shape")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == k_cache.dtype and t.device == k_cache.device and t.is_contiguous(),
                 f"{name} must be contiguous, on {k_cache.device}, dtype {k_cache.dtype}")
    _require(k_new.numel() == B * Hkv * D and v_new.numel() == B * Hkv * D, "k_new/v_new must be [B, Hkv, D]")
    _require(k_cache.dtype in _DTYPE_CODES, "dtype must be float16 or bfloat16")
    pos_t = _as_int32(pos, B, k_cache.device)
    _check(_lib.ada_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(pos_t), B, Hkv, S, D,
                              _DTYPE_CODES[k_cache.dtype], ctypes.c_void_p(_stream(k_cache.device))),
           "ada_kv_append")


def _lengths(kv_len, max_kv_len, batch: int, capacity: int, device):
    """(device lengths or None, max_kv_len) for the C call. A host int, or host
    ints all equal, become the lockstep form (NULL lengths, max_kv_len = that
    value, clamped to [0, capacity]); ``None`` means every row holds
    ``max_kv_len`` slots; a device tensor is passed as is (``max_kv_len``
    defaults to the capacity); other host lists are copied to the device."""
    if isinstance(kv_len, torch.Tensor):
        return _as_int32(kv_len, batch, device), (capacity if max_kv_len is None else int(max_kv_len))
    if kv_len is None:
        _require(max_kv_len is not None, "kv_len=None needs max_kv_len")
        return None, int(max_kv_len)
    host = [int(v) for v in (kv_len if hasattr(kv_len, "__len__") else [kv_len] * batch)]
    _require(len(host) == batch, "need one kv_len per batch row")
    if host and all(v == host[0] for v in host) and max_kv_len is None and host[0] > 0:
        # (an all-empty batch keeps the device form: max_kv_len <= 0 means "capacity")
        return None, min(capacity, host[0])
    mkl = max(1, min(capacity, max(host) if host else 1)) if max_kv_len is None else int(max_kv_len)
    return _as_int32(host, batch, device), mkl


def _as_int32(x, batch: int, device) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        _require(x.dtype == torch.int32 and x.is_cuda and x.is_contiguous() and x.numel() == batch,
                 "index tensors must be contiguous int32 GPU tensors with one entry per batch row")
        return x
    vals = [int(v) for v in (x if hasattr(x, "__len__") else [x] * batch)]
    _require(len(vals) == batch, "need one entry per batch row")
    return torch.tensor(vals, dtype=torch.int32, device=device)


def decode_attn_gqa_ex(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len,
                       scale: float | None = None, out: torch.Tensor | None = None,
                       max_kv_len: int | None = None, num_splits: int = 0,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention with a forced split count (0 = heuristic)."""
    _require(k_cache.is_cuda and k_cache.dim() == 4, "k_cache must be a 4-d GPU tensor [B, Hkv, S, D]")
    B, Hkv, S, D = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "v_cache shape must equal k_cache shape")
    _require(q.dim() in (3, 4) and q.shape[0] == B and q.shape[-1] == D and (q.dim() == 3 or q.shape[2] == 1),
             "q must be [B, Hq, D] or [B, Hq, 1, D]")
    Hq = q.shape[1]
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == k_cache.dtype and t.device == k_cache.device and t.is_contiguous(),
                 f"{name} must be contiguous, on {k_cache.device}, dtype {k_cache.dtype}")
    _require(k_cache.dtype in _DTYPE_CODES, "dtype must be float16 or bfloat16")
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.device == q.device and out.is_contiguous(),
             "out must be a contiguous tensor like q")
    lens_t, mkl = _lengths(kv_len, max_kv_len, B, S, k_cache.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    plan_len = S if mkl <= 0 else min(mkl, S)  # the library reads max_kv_len <= 0 as the capacity
    splits, _ = decode_plan(B, Hq, Hkv, plan_len, num_splits)
    need = decode_workspace_bytes(B, Hq, Hkv, D, splits) if splits > 1 else 0
    ws = workspace if workspace is not None else _workspace(k_cache.device, need)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    rc = _lib.ada_decode_attn_gqa_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens_t), B, Hq, Hkv, D, S, mkl,
                                     ctypes.c_float(scale), _DTYPE_CODES[k_cache.dtype], _ptr(out), _ptr(ws),
                                     ws_bytes, ctypes.c_void_p(_stream(k_cache.device)), int(num_splits))
    _check(rc, "ada_decode_attn_gqa_ex")
    return out


def _check_decode_inputs(q, k_cache, v_cache):
    _require(k_cache.is_cuda and k_cache.dim() == 4, "k_cache must be a 4-d GPU tensor [B, Hkv, S, D]")
    B, Hkv, S, D = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "v_cache shape must equal k_cache shape")
    _require(q.dim() in (3, 4) and q.shape[0] == B and q.shape[-1] == D and (q.dim() == 3 or q.shape[2] == 1),
             "q must be [B, Hq, D] or [B, Hq, 1, D]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == k_cache.dtype and t.device == k_cache.device and t.is_contiguous(),
                 f"{name} must be contiguous, on {k_cache.device}, dtype {k_cache.dtype}")
    _require(k_cache.dtype in _DTYPE_CODES, "dtype must be float16 or bfloat16")
    return B, q.shape[1], Hkv, S, D


def workspace_layout(batch: int, n_head: int, num_splits: int, head_dim: int = HEAD_DIM) -> dict:
    """Byte offsets of the split-major partials in a workspace (as include/ada.h
    documents them): float2 (m, l) per (split, batch row, query head) from
    ``ml_offset``, float[head_dim] accumulators from ``acc_offset``."""
    r256 = lambda x: (x + 255) // 256 * 256
    rows = batch * n_head * num_splits
    acc_offset = r256(rows * 8)
    return {"ml_offset": 0, "acc_offset": acc_offset, "total": acc_offset + r256(rows * head_dim * 4),
            "rows_per_split": batch * n_head}


def decode_partial(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len,
                   scale: float | None = None, max_kv_len: int | None = None, num_splits: int = 0,
                   workspace: torch.Tensor | None = None):
    """First half of a decode call: per-split partial results (running max, sum
    and unnormalised accumulator, split-major) written to ``workspace``.
    Returns ``(workspace, splits_used)``."""
    B, Hq, Hkv, S, D = _check_decode_inputs(q, k_cache, v_cache)
    lens_t, mkl = _lengths(kv_len, max_kv_len, B, S, k_cache.device)
    plan_len = S if mkl <= 0 else min(mkl, S)
    splits, _ = decode_plan(B, Hq, Hkv, plan_len, num_splits)
    if workspace is None:
        workspace = new_workspace(decode_workspace_bytes(B, Hq, Hkv, D, splits), k_cache.device)
    used = ctypes.c_int(0)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = _lib.ada_decode_partial(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens_t), B, Hq, Hkv, D, S, mkl,
                                 ctypes.c_float(scale), _DTYPE_CODES[k_cache.dtype], int(num_splits), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), ctypes.byref(used),
                                 ctypes.c_void_p(_stream(k_cache.device)))
    _check(rc, "ada_decode_partial")
    return workspace, used.value


def decode_combine(workspace: torch.Tensor, num_splits: int, out: torch.Tensor, n_kv_head: int) -> torch.Tensor:
    """Second half of a decode call: merge ``num_splits`` split-major partials
    in ``workspace`` into ``out`` [B, Hq, D] (or [B, Hq, 1, D])."""
    _require(out.is_cuda and out.is_contiguous() and out.dtype in _DTYPE_CODES, "out must be a contiguous 16-bit GPU tensor")
    _require(workspace.is_cuda and workspace.device == out.device, "workspace must be on the output's device")
    B, Hq, D = out.shape[0], out.shape[1], out.shape[-1]
    rc = _lib.ada_decode_combine(_ptr(workspace), workspace.numel() * workspace.element_size(), B, Hq, int(n_kv_head),
                                 D, int(num_splits), _DTYPE_CODES[out.dtype], _ptr(out),
                                 ctypes.c_void_p(_stream(out.device)))
    _check(rc, "ada_decode_combine")
    return out


def decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                v_cache: torch.Tensor, pos, scale: float | None = None, out: torch.Tensor | None = None,
                max_pos: int | None = None, num_splits: int = 0,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one call: write k_new/v_new [B, Hkv, D] at slot pos
    of the caches, then attend over slots 0..pos (kv_len = pos + 1). ``pos``:
    a host int (every row at that slot), host ints, or an int32 GPU tensor
    (then ``max_pos`` bounds it, default the last slot)."""
    return _decode_step(q, k_new, v_new, None, None, k_cache, v_cache, pos, scale, out, max_pos, num_splits,
                        workspace)


def decode_step_rope(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cos: torch.Tensor,
                     sin: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, pos, scale: float | None = None,
                     out: torch.Tensor | None = None, max_pos: int | None = None, num_splits: int = 0,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode_step with the rotary embedding of ``rope_kv_append`` applied to q
    and k_new first (cos / sin: [B, D] tables in the cache dtype, row b for
    batch row b's position). q is not modified."""
    return _decode_step(q, k_new, v_new, cos, sin, k_cache, v_cache, pos, scale, out, max_pos, num_splits,
                        workspace)


def _check_tables(cos, sin, B, D, like):
    for name, t in (("cos", cos), ("sin", sin)):
        _require(isinstance(t, torch.Tensor) and t.dtype == like.dtype and t.device == like.device
                 and t.is_contiguous() and t.numel() == B * D,
                 f"{name} must be a contiguous [B, D] tensor in {like.dtype} on {like.device}")


def rope_kv_append(q, k_new: torch.Tensor, v_new: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, pos, q_out: torch.Tensor | None = None):
    """Rotate q [B, Hq, D] into q_out (allocated when None; may be q itself)
    and k_new [B, Hkv, D] with the rotate-half rotary map, then write the
    rotated key and v_new at slot pos[b] of the caches [B, Hkv, S, D]. ``q``
    may be None (keys only). ``pos``: int32 GPU tensor [B] or host ints.
    Returns q_out (None when q is None)."""
    _require(k_cache.is_cuda and k_cache.dim() == 4, "k_cache must be a 4-d GPU tensor [B, Hkv, S, D]")
    B, Hkv, S, D = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "v_cache shape must equal k_cache shape")
    _require(k_cache.dtype in _DTYPE_CODES, "dtype must be float16 or bfloat16")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == k_cache.dtype and t.device == k_cache.device and t.is_contiguous(),
                 f"{name} must be contiguous, on {k_cache.device}, dtype {k_cache.dtype}")
    _require(k_new.numel() == B * Hkv * D and v_new.numel() == B * Hkv * D, "k_new/v_new must be [B, Hkv, D]")
    _check_tables(cos, sin, B, D, k_cache)
    Hq = 0
    if q is not None:
        _require(q.dtype == k_cache.dtype and q.device == k_cache.device and q.is_contiguous()
                 and q.shape[0] == B and q.shape[-1] == D and q.numel() % (B * D) == 0,
                 "q must be a contiguous [B, Hq, D] tensor like the cache")
        Hq = q.numel() // (B * D)
        if q_out is None:
            q_out = torch.empty_like(q)
        _require(q_out.shape == q.shape and q_out.dtype == q.dtype and q_out.is_contiguous(), "q_out must be like q")
    pos_t = _as_int32(pos, B, k_cache.device)
    _check(_lib.ada_rope_kv_append(_ptr(q), _ptr(q_out), _ptr(k_new), _ptr(v_new), _ptr(cos), _ptr(sin),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(pos_t), B, Hq, Hkv, S, D,
                                   _DTYPE_CODES[k_cache.dtype], ctypes.c_void_p(_stream(k_cache.device))),
           "ada_rope_kv_append")
    return q_out


def _start_arg(start, batch: int, device):
    """None or 0 -> NULL (every row from slot 0); else an int32 device tensor."""
    if start is None or (not isinstance(start, torch.Tensor) and not hasattr(start, "__len__") and int(start) == 0):
        return None
    if not isinstance(start, torch.Tensor) and not hasattr(start, "__len__"):
        start = [int(start)] * batch
    return _as_int32(start, batch, device)


def prefill_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   start=None) -> None:
    """Write the prompt rows k_new/v_new [B, Hkv, T, D] into slots start[b] ..
    start[b] + T - 1 of the caches [B, Hkv, S, D], in place. ``start``: None
    (slot 0), a host int or ints, or an int32 GPU tensor [B]."""
    _require(k_cache.is_cuda and k_cache.dim() == 4, "k_cache must be a 4-d GPU tensor [B, Hkv, S, D]")
    B, Hkv, S, D = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "v_cache shape must equal k_cache shape")
    _require(k_cache.dtype in _DTYPE_CODES, "dtype must be float16 or bfloat16")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == k_cache.dtype and t.device == k_cache.device and t.is_contiguous(),
                 f"{name} must be contiguous, on {k_cache.device}, dtype {k_cache.dtype}")
    _require(k_new.dim() == 4 and k_new.shape[:2] == (B, Hkv) and k_new.shape[3] == D and v_new.shape == k_new.shape,
             "k_new/v_new must be [B, Hkv, T, D]")
    T = k_new.shape[2]
    st = _start_arg(start, B, k_cache.device)
    _check(_lib.ada_prefill_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(st), B, Hkv, T, S, D,
                                   _DTYPE_CODES[k_cache.dtype], ctypes.c_void_p(_stream(k_cache.device))),
           "ada_prefill_append")


def prefill_attn_gqa(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, start=None,
                     scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal prefill attention: q [B, Hq, T, D]; token t of row b attends cache
    slots 0 .. start[b] + t (start None = 0: SDPA with is_causal=True over the
    prompt). Returns out [B, Hq, T, D]."""
    _require(q.is_cuda and q.dim() == 4, "q must be a 4-d GPU tensor [B, Hq, T, D]")
    _require(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [B, Hkv, S, D]")
    B, Hq, T, D = q.shape
    _, Hkv, S, _ = k_cache.shape
    _require(k_cache.shape[0] == B and k_cache.shape[3] == D, "q and caches disagree")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == q.dtype and t.device == q.device and t.is_contiguous(),
                 f"{name} must be contiguous, on {q.device}, dtype {q.dtype}")
    _require(q.dtype in _DTYPE_CODES, "dtype must be float16 or bfloat16")
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "out must be like q")
    st = _start_arg(start, B, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_lib.ada_prefill_attn_gqa(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(st), B, Hq, Hkv, T, D, S,
                                     ctypes.c_float(scale), _DTYPE_CODES[q.dtype], _ptr(out),
                                     ctypes.c_void_p(_stream(q.device))),
           "ada_prefill_attn_gqa")
    return out


def _decode_step(q, k_new, v_new, cos, sin, k_cache, v_cache, pos, scale, out, max_pos, num_splits, workspace):
    B, Hq, Hkv, S, D = _check_decode_inputs(q, k_cache, v_cache)
    if cos is not None or sin is not None:
        _check_tables(cos, sin, B, D, k_cache)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _require(t.dtype == k_cache.dtype and t.device == k_cache.device and t.is_contiguous()
                 and t.numel() == B * Hkv * D, f"{name} must be a contiguous [B, Hkv, D] tensor like the cache")
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "out must be like q")
    if isinstance(pos, torch.Tensor):
        pos_t = _as_int32(pos, B, k_cache.device)
        mp = S - 1 if max_pos is None else int(max_pos)
    else:
        host = [int(v) for v in (pos if hasattr(pos, "__len__") else [pos] * B)]
        _require(len(host) == B, "need one position per batch row")
        if all(v == host[0] for v in host) and max_pos is None and 0 <= host[0] < S:
            pos_t, mp = None, host[0]
        else:
            pos_t = _as_int32(host, B, k_cache.device)
            mp = max(0, min(S - 1, max(host))) if max_pos is None else int(max_pos)
    plan_len = min(mp + 1, S)
    splits, _ = decode_plan(B, Hq, Hkv, plan_len, num_splits)
    need = decode_workspace_bytes(B, Hq, Hkv, D, splits) if splits > 1 else 0
    ws = workspace if workspace is not None else _workspace(k_cache.device, need)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if cos is None:
        rc = _lib.ada_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(pos_t), B,
                                  Hq, Hkv, D, S, mp, ctypes.c_float(scale), _DTYPE_CODES[k_cache.dtype], _ptr(out),
                                  _ptr(ws), ws_bytes, ctypes.c_void_p(_stream(k_cache.device)), int(num_splits))
        _check(rc, "ada_decode_step")
    else:
        rc = _lib.ada_decode_step_rope(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cos), _ptr(sin), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(pos_t), B, Hq, Hkv, D, S, mp, ctypes.c_float(scale),
                                       _DTYPE_CODES[k_cache.dtype], _ptr(out), _ptr(ws), ws_bytes,
                                       ctypes.c_void_p(_stream(k_cache.device)), int(num_splits))
        _check(rc, "ada_decode_step_rope")
    return out


class StepGraph:
    """A whole multi-layer decode step recorded once as a HIP graph by
    ``ada_step_graph_create``; ``launch()`` replays it on the current stream.
    Holds references to every buffer it was built on, so they outlive it."""

    def __init__(self, handle: int, device: torch.device, keep: tuple):
        self._handle = handle
        self.device = device
        self._keep = keep

    def launch(self) -> None:
        _require(self._handle is not None, "step graph is closed")
        _check(_lib.ada_step_graph_launch(ctypes.c_void_p(self._handle), ctypes.c_void_p(_stream(self.device))),
               "ada_step_graph_launch")

    def close(self) -> None:
        """Free the graph; synchronise the streams it was launched on first."""
        if self._handle is not None:
            _lib.ada_step_graph_destroy(ctypes.c_void_p(self._handle))
            self._handle = None
            self._keep = ()

    def __del__(self):
        try:
            if self._handle is not None:
                torch.cuda.synchronize(self.device)
            self.close()
        except Exception:
            pass


def step_graph(layers, pos: torch.Tensor, max_pos: int, scale: float | None = None, advance: bool = True,
               workspace: torch.Tensor | None = None) -> StepGraph:
    """Record one decode step of every layer, in order, then the advance
    pos[b] += 1 (when ``advance``), as one HIP graph.

    ``layers``: a sequence of (q, k_new, v_new, k_cache, v_cache, out) or
    (q, k_new, v_new, k_cache, v_cache, out, cos, sin) tuples, all layers with
    the same cache shape and dtype; ``pos``: int32 GPU tensor [B];
    ``max_pos``: the largest position any launch will see (sizes the
    launches). Each launch of the returned graph runs ``decode_step`` (or
    ``decode_step_rope``) on every layer with these buffers' current
    contents."""
    layers = list(layers)
    _require(len(layers) > 0, "need at least one layer")
    k0 = layers[0][3]
    B, Hq, Hkv, S, D = _check_decode_inputs(layers[0][0], k0, layers[0][4])
    dev = k0.device
    pos_t = _as_int32(pos, B, dev)
    _require(isinstance(pos, torch.Tensor), "pos must be an int32 GPU tensor (the graph advances it in place)")
    structs = (StepLayer * len(layers))()
    keep = [pos_t]
    for i, layer in enumerate(layers):
        _require(len(layer) in (6, 8), "a layer is (q, k_new, v_new, k_cache, v_cache, out[, cos, sin])")
        q, k_new, v_new, kc, vc, out = layer[:6]
        cos, sin = (layer[6], layer[7]) if len(layer) == 8 else (None, None)
        _require(kc.shape == k0.shape and kc.dtype == k0.dtype and kc.device == dev,
                 "every layer's caches must match the first layer's shape, dtype and device")
        _check_decode_inputs(q, kc, vc)
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            _require(t.dtype == kc.dtype and t.device == dev and t.is_contiguous() and t.numel() == B * Hkv * D,
                     f"{name} must be a contiguous [B, Hkv, D] tensor like the cache")
        _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "out must be like q")
        if cos is not None or sin is not None:
            _check_tables(cos, sin, B, D, kc)
        structs[i] = StepLayer(*(t.data_ptr() if t is not None else None for t in (q, k_new, v_new, kc, vc, out, cos, sin)))
        keep.append(tuple(layer))
    mp = int(max_pos)
    splits = decode_num_splits(B, Hq, Hkv, min(mp + 1, S)) if 0 <= mp < S else 1
    if workspace is None and splits > 1:
        workspace = new_workspace(decode_workspace_bytes(B, Hq, Hkv, D, splits), dev)
    keep.append(workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    handle = ctypes.c_void_p(0)
    _check(_lib.ada_step_graph_create(structs, len(layers), _ptr(pos_t), B, Hq, Hkv, D, S, mp, ctypes.c_float(scale),
                                      _DTYPE_CODES[k0.dtype], 1 if advance else 0, _ptr(workspace), ws_bytes,
                                      ctypes.byref(handle)), "ada_step_graph_create")
    return StepGraph(handle.value, dev, tuple(keep))


def hbm_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int) -> None:
    """Measurement: stream every byte of ``src`` (contiguous, 16-byte
    aligned, size a multiple of 16) once on the current stream with the
    decode kernel's loads; ``sink`` (uint32-sized, >= 4 * workgroups entries)
    receives one xor per wavefront."""
    _require(src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.is_contiguous(),
             "src and sink must be contiguous GPU tensors")
    nbytes = src.numel() * src.element_size()
    _require(sink.numel() * sink.element_size() >= 16 * workgroups, "sink needs 4 * workgroups uint32 entries")
    _check(_lib.ada_hbm_read(_ptr(src), nbytes, _ptr(sink), int(workgroups), ctypes.c_void_p(_stream(src.device))),
           "ada_hbm_read")


def decode_attn_gqa_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len,
                            scale: float | None = None, out: torch.Tensor | None = None,
                            max_kv_len: int | None = None, num_splits: int = 0) -> torch.Tensor:
    """``decode_attn_gqa_ex`` through ``ada_decode_attn_gqa_noalloc``: the split
    partials go to the library's static per-device scratch buffer, so the call
    allocates no device memory (``out`` must then be given by a caller that
    cannot allocate; host lengths are still copied to the device here, so such
    a caller passes an int32 GPU tensor or one host length). Calls on one
    device must not overlap (they share the buffer)."""
    B, Hq, Hkv, S, D = _check_decode_inputs(q, k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.device == q.device and out.is_contiguous(),
             "out must be a contiguous tensor like q")
    lens_t, mkl = _lengths(kv_len, max_kv_len, B, S, k_cache.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_lib.ada_decode_attn_gqa_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens_t), B, Hq, Hkv, D, S,
                                            mkl, ctypes.c_float(scale), _DTYPE_CODES[k_cache.dtype], _ptr(out),
                                            ctypes.c_void_p(_stream(k_cache.device)), int(num_splits)),
           "ada_decode_attn_gqa_noalloc")
    return out


def decode_attn_gqa(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len,
                    scale: float | None = None, out: torch.Tensor | None = None,
                    max_kv_len: int | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """out = softmax(scale * q K[:kv_len]^T) V[:kv_len] per batch row, grouped-query
    heads read in place (query head h uses KV head h // (Hq // Hkv)).

    q: [B, Hq, D] or [B, Hq, 1, D]; caches [B, Hkv, S, D]; kv_len: int32 GPU
    tensor [B] (then ``max_kv_len`` bounds it, default S) or host ints. Returns
    ``out`` (allocated like q when not given). Runs on the current stream."""
    return decode_attn_gqa_ex(q, k_cache, v_cache, kv_len, scale=scale, out=out, max_kv_len=max_kv_len,
                              num_splits=0, workspace=workspace)


__all__ = [
    "AdaError", "F16", "BF16", "HEAD_DIM", "MAX_SPLITS", "EXPORTS", "LIB_PATH", "load_library",
    "kv_append", "decode_attn_gqa", "decode_attn_gqa_ex", "decode_attn_gqa_noalloc", "decode_partial", "decode_combine", "decode_step", "decode_step_rope",
    "rope_kv_append", "prefill_append", "prefill_attn_gqa", "decode_num_splits", "decode_plan", "decode_workspace_bytes",
    "new_workspace", "workspace_layout", "device_num_cus", "status_string", "last_hip_error",
    "abi_version", "StepGraph", "StepLayer", "step_graph", "prefill_rows_per_workgroup", "hbm_read",
]
