"""bitmask_spmv_amd -- N:M bitmask sparse decode kernels for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``include/nm_spmv.h`` (``libnmspmv.so``, built
in-tree by ``bitmask_spmv_amd._build``).  Every function has the C entry point's name
and only marshals arguments: it checks dtypes, devices, shapes and strides of torch
tensors, passes their device pointers and the current HIP stream, and turns a
non-zero status into :class:`NmError`.  All arithmetic runs in the HIP kernels; there
is no CPU fallback, and importing this package fails loudly when the library has not
been built.

PyTorch is used only for device memory and streams.  ``masks`` are carried in int32
tensors that hold the raw uint32 mask words; bf16 tensors are passed as raw patterns.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "NmError", "LIB_PATH", "lib", "nm_version", "nm_col_norm", "nm_prune_pack", "nm_spmv",
    "nm_spmv_workspace_bytes", "dense_gemv", "dense_gemv_workspace_bytes", "nm_unpack",
    "NM_PATTERNS", "nm_spmv_multi", "nm_spmv_multi_workspace_bytes", "dense_gemv_multi",
    "dense_gemv_multi_workspace_bytes", "NM_META_BITMASK", "NM_META_U8_OFFSET", "NM_META_I32_INDEX",
    "nm_meta_from_mask", "nm_spmv_meta", "nm_spmv_swiglu", "nm_spmv_swiglu_workspace_bytes", "dense_gemv_swiglu",
    "dense_gemv_swiglu_workspace_bytes", "nm_prune_pack_unstructured", "nm_spmv_unstructured",
    "nm_spmv_unstructured_workspace_bytes", "nm_unpack_unstructured", "nm_hessian", "nm_obs_inverse_factor",
    "nm_obs_inverse_factor_workspace_bytes", "nm_sparsegpt_prune_pack", "nm_sparsegpt_workspace_bytes",
    "nm_stream_read", "nm_stream_read_sink_words", "nm_spmv_plan", "nm_spmv_multi_plan", "NM_EPI_NONE",
    "NM_EPI_SWIGLU", "NM_KERNEL_WORD", "NM_KERNEL_TILE", "NM_KERNEL_WORD_HALF_ROWS", "NM_KERNEL_WORD_STRIPS",
    "nm_spmv_noalloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnmspmv.so")
NM_PATTERNS = ((2, 4), (4, 8), (8, 16), (16, 32))
NM_META_BITMASK, NM_META_U8_OFFSET, NM_META_I32_INDEX = 0, 1, 2
NM_EPI_NONE, NM_EPI_SWIGLU = 0, 1
NM_KERNEL_WORD, NM_KERNEL_TILE, NM_KERNEL_WORD_HALF_ROWS, NM_KERNEL_WORD_STRIPS = 0, 1, 2, 3

_STATUS = {0: "NM_OK", 1: "NM_ERR_NULL", 2: "NM_ERR_SHAPE", 3: "NM_ERR_PATTERN", 4: "NM_ERR_ALIGN",
           5: "NM_ERR_WORKSPACE", 6: "NM_ERR_HIP"}


class NmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")


class _SpmvMatrix(ctypes.Structure):
    _fields_ = [("masks", ctypes.c_void_p), ("values", ctypes.c_void_p), ("R", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


class _LaunchPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("threads", ctypes.c_int), ("grid_x", ctypes.c_int),
                ("splits", ctypes.c_int), ("tiles_per_step", ctypes.c_int), ("x_steps_in_registers", ctypes.c_int),
                ("rows_per_group", ctypes.c_int), ("lds_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]


class _DenseMatrix(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("ldw", ctypes.c_int64), ("R", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or python bitmask_spmv_amd/_build.py); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    i64, p, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.nm_status_str.argtypes, L.nm_status_str.restype = [i32], ctypes.c_char_p
    L.nm_last_error.argtypes, L.nm_last_error.restype = [], ctypes.c_char_p
    L.nm_version.argtypes, L.nm_version.restype = [], i32
    L.nm_col_norm.argtypes = [p, i64, i64, i64, p, p]
    L.nm_prune_pack.argtypes = [p, i64, i64, i64, p, i32, i32, p, p, p]
    L.nm_spmv_workspace_bytes.argtypes, L.nm_spmv_workspace_bytes.restype = [i64, i64, i32], sz
    L.nm_spmv.argtypes = [p, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.nm_spmv_noalloc.argtypes, L.nm_spmv_noalloc.restype = [p, p, i64, i64, p, i64, i32, p, i64, p], i32
    L.dense_gemv_workspace_bytes.argtypes, L.dense_gemv_workspace_bytes.restype = [i64, i64, i32], sz
    L.dense_gemv.argtypes = [p, i64, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.nm_unpack.argtypes = [p, p, i64, i64, p, i64, p]
    L.nm_meta_from_mask.argtypes = [p, i64, i64, i32, p, p]
    f64 = ctypes.c_double
    L.nm_hessian.argtypes = [p, i64, i64, i64, p, i64, p]
    L.nm_obs_inverse_factor_workspace_bytes.argtypes = [i64]
    L.nm_obs_inverse_factor_workspace_bytes.restype = sz
    L.nm_obs_inverse_factor.argtypes = [p, i64, i64, f64, p, i64, p, sz, p]
    L.nm_sparsegpt_workspace_bytes.argtypes = [i64, i64]
    L.nm_sparsegpt_workspace_bytes.restype = sz
    L.nm_sparsegpt_prune_pack.argtypes = [p, i64, i64, i64, p, i64, i32, i32, f64, p, p, p, sz, p]
    L.nm_prune_pack_unstructured.argtypes = [p, i64, i64, i64, p, p, p, p]
    L.nm_spmv_unstructured_workspace_bytes.argtypes = [i64, i64, i32]
    L.nm_spmv_unstructured_workspace_bytes.restype = sz
    L.nm_spmv_unstructured.argtypes = [p, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.nm_unpack_unstructured.argtypes = [p, p, i64, i64, p, i64, p]
    L.nm_spmv_swiglu_workspace_bytes.argtypes, L.nm_spmv_swiglu_workspace_bytes.restype = [i64, i64, i32], sz
    L.nm_spmv_swiglu.argtypes = [p, p, p, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.dense_gemv_swiglu_workspace_bytes.argtypes, L.dense_gemv_swiglu_workspace_bytes.restype = [i64, i64, i32], sz
    L.dense_gemv_swiglu.argtypes = [p, p, i64, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.nm_spmv_meta.argtypes = [p, i32, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.nm_spmv_multi_workspace_bytes.argtypes = [p, i32, i64, i32]
    L.nm_spmv_multi_workspace_bytes.restype = sz
    L.nm_spmv_multi.argtypes = [p, i32, i64, p, i64, i32, p, sz, p]
    L.dense_gemv_multi_workspace_bytes.argtypes = [p, i32, i64, i32]
    L.dense_gemv_multi_workspace_bytes.restype = sz
    L.dense_gemv_multi.argtypes = [p, i32, i64, p, i64, i32, p, sz, p]
    L.nm_stream_read_sink_words.argtypes, L.nm_stream_read_sink_words.restype = [sz], sz
    L.nm_stream_read.argtypes, L.nm_stream_read.restype = [p, sz, p, sz, p], i32
    L.nm_spmv_plan.argtypes, L.nm_spmv_plan.restype = [i64, i64, i32, i32, p], i32
    L.nm_spmv_multi_plan.argtypes, L.nm_spmv_multi_plan.restype = [p, i32, i64, i32, p], i32
    for f in (L.nm_col_norm, L.nm_prune_pack, L.nm_spmv, L.dense_gemv, L.nm_unpack, L.nm_spmv_multi,
              L.dense_gemv_multi):
        f.restype = i32
    return L


lib = _load()


def _check(status: int):
    if status != 0:
        raise NmError(status, lib.nm_last_error().decode(errors="replace"))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a HIP device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous in its last dimension")


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.dim() == 2 and t.shape[0] > 1 else t.shape[-1]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def nm_version() -> int:
    return int(lib.nm_version())


def nm_col_norm(X: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """X: bf16 [T, K] calibration activations -> fp32 [K] column norms."""
    _dev(X, "X", torch.bfloat16, 2)
    T, K = X.shape
    if out is None:
        out = torch.empty(K, dtype=torch.float32, device=X.device)
    _dev(out, "out", torch.float32, 1)
    _check(lib.nm_col_norm(_ptr(X), T, K, _ld(X), _ptr(out), _stream(X)))
    return out


def nm_prune_pack(W: torch.Tensor, col_norm: torch.Tensor, N: int, M: int, masks: torch.Tensor | None = None,
                  values: torch.Tensor | None = None):
    """W: bf16 [R, K]; col_norm: fp32 [K] -> (masks int32 [R, K/32], values bf16 [R, K/2])."""
    _dev(W, "W", torch.bfloat16, 2)
    _dev(col_norm, "col_norm", torch.float32, 1)
    R, K = W.shape
    if col_norm.shape[0] != K:
        raise ValueError("col_norm must have K entries")
    if masks is None:
        masks = torch.empty((R, max(K // 32, 1)), dtype=torch.int32, device=W.device)
    if values is None:
        values = torch.empty((R, max(K // 2, 1)), dtype=torch.bfloat16, device=W.device)
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    if not (masks.is_contiguous() and values.is_contiguous()):
        raise ValueError("masks and values must be contiguous")
    if K % 32 == 0 and (masks.shape != (R, K // 32) or values.shape != (R, K // 2)):
        raise ValueError("masks must be [R, K/32] and values [R, K/2]")
    _check(lib.nm_prune_pack(_ptr(W), _ld(W), R, K, _ptr(col_norm), int(N), int(M), _ptr(masks), _ptr(values),
                             _stream(W)))
    return masks, values


def nm_spmv_workspace_bytes(R: int, K: int, B: int) -> int:
    return int(lib.nm_spmv_workspace_bytes(R, K, B))


def dense_gemv_workspace_bytes(R: int, K: int, B: int) -> int:
    return int(lib.dense_gemv_workspace_bytes(R, K, B))


def _workspace(nbytes: int, ref: torch.Tensor, workspace: torch.Tensor | None):
    if nbytes == 0:
        return workspace, 0
    if workspace is None:
        workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=ref.device)
    if workspace.device != ref.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    return workspace, workspace.numel() * workspace.element_size()


def _x_y(x: torch.Tensor, R: int, K: int, out: torch.Tensor | None):
    squeeze = x.dim() == 1
    if squeeze:
        x = x.unsqueeze(0)
    _dev(x, "x", torch.bfloat16, 2)
    B = x.shape[0]
    if x.shape[1] != K:
        raise ValueError(f"x has {x.shape[1]} columns, expected K={K}")
    if out is None:
        out = torch.empty((B, R), dtype=torch.bfloat16, device=x.device)
    o2 = out.unsqueeze(0) if out.dim() == 1 else out
    _dev(o2, "out", torch.bfloat16, 2)
    if o2.shape != (B, R):
        raise ValueError(f"out must be [{B}, {R}]")
    return x, B, o2, out, squeeze


def nm_spmv(masks: torch.Tensor, values: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = W_sparse x for packed (masks, values); x: bf16 [B, K] or [K] -> bf16 [B, R] (or [R])."""
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    if not (masks.is_contiguous() and values.is_contiguous()):
        raise ValueError("masks and values must be contiguous")
    R = masks.shape[0]
    K = masks.shape[1] * 32
    if values.shape != (R, K // 2):
        raise ValueError("values must be [R, K/2] with K = 32 * masks.shape[1]")
    x2, B, o2, out, squeeze = _x_y(x, R, K, out)
    ws, ws_bytes = _workspace(nm_spmv_workspace_bytes(R, K, B), x2, workspace)
    _check(lib.nm_spmv(_ptr(masks), _ptr(values), R, K, _ptr(x2), _ld(x2), B, _ptr(o2), _ld(o2), _ptr(ws),
                       ws_bytes, _stream(x2)))
    return out[0] if squeeze and out.dim() == 2 else out


def nm_spmv_noalloc(masks: torch.Tensor, values: torch.Tensor, x: torch.Tensor,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """nm_spmv without a workspace: split rows use the library's fixed per-device scratch.
    Allocates nothing when `out` is given."""
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    if not (masks.is_contiguous() and values.is_contiguous()):
        raise ValueError("masks and values must be contiguous")
    R = masks.shape[0]
    K = masks.shape[1] * 32
    if values.shape != (R, K // 2):
        raise ValueError("values must be [R, K/2] with K = 32 * masks.shape[1]")
    x2, B, o2, out, squeeze = _x_y(x, R, K, out)
    _check(lib.nm_spmv_noalloc(_ptr(masks), _ptr(values), R, K, _ptr(x2), _ld(x2), B, _ptr(o2), _ld(o2),
                               _stream(x2)))
    return out[0] if squeeze and out.dim() == 2 else out


def dense_gemv(W: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x; W: bf16 [R, K]; x: bf16 [B, K] or [K] -> bf16 [B, R] (or [R])."""
    _dev(W, "W", torch.bfloat16, 2)
    R, K = W.shape
    x2, B, o2, out, squeeze = _x_y(x, R, K, out)
    ws, ws_bytes = _workspace(dense_gemv_workspace_bytes(R, K, B), x2, workspace)
    _check(lib.dense_gemv(_ptr(W), _ld(W), R, K, _ptr(x2), _ld(x2), B, _ptr(o2), _ld(o2), _ptr(ws), ws_bytes,
                          _stream(x2)))
    return out[0] if squeeze and out.dim() == 2 else out


def nm_unpack(masks: torch.Tensor, values: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Packed (masks, values) -> dense pruned bf16 [R, K] (zeros where bits are clear)."""
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    R = masks.shape[0]
    K = masks.shape[1] * 32
    if out is None:
        out = torch.empty((R, K), dtype=torch.bfloat16, device=masks.device)
    _dev(out, "out", torch.bfloat16, 2)
    _check(lib.nm_unpack(_ptr(masks), _ptr(values), R, K, _ptr(out), _ld(out), _stream(masks)))
    return out


def _meta_shape(fmt: int, R: int, K: int):
    if fmt == NM_META_BITMASK:
        return torch.int32, (R, K // 32)
    if fmt == NM_META_U8_OFFSET:
        return torch.uint8, (R, K // 2)
    if fmt == NM_META_I32_INDEX:
        return torch.int32, (R, K // 2)
    raise ValueError(f"unknown metadata format {fmt}")


def nm_meta_from_mask(masks: torch.Tensor, fmt: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Canonical masks int32 [R, K/32] -> uint8 offsets [R, K/2] (NM_META_U8_OFFSET) or int32
    column indices [R, K/2] (NM_META_I32_INDEX), in the order of the packed values."""
    _dev(masks, "masks", torch.int32, 2)
    if not masks.is_contiguous():
        raise ValueError("masks must be contiguous")
    R, K = masks.shape[0], masks.shape[1] * 32
    if fmt not in (NM_META_U8_OFFSET, NM_META_I32_INDEX):
        raise ValueError("fmt must be NM_META_U8_OFFSET or NM_META_I32_INDEX")
    dtype, shape = _meta_shape(fmt, R, K)
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=masks.device)
    _dev(out, "out", dtype, 2)
    if out.shape != shape or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dtype} tensor of shape {shape}")
    _check(lib.nm_meta_from_mask(_ptr(masks), R, K, int(fmt), _ptr(out), _stream(masks)))
    return out


def nm_spmv_meta(meta: torch.Tensor, fmt: int, values: torch.Tensor, x: torch.Tensor,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """nm_spmv with metadata in any format: masks int32 [R, K/32] (NM_META_BITMASK), uint8 offsets
    [R, K/2] (NM_META_U8_OFFSET) or int32 column indices [R, K/2] (NM_META_I32_INDEX)."""
    _dev(values, "values", torch.bfloat16, 2)
    R, K = values.shape[0], values.shape[1] * 2
    dtype, shape = _meta_shape(fmt, R, K)
    _dev(meta, "meta", dtype, 2)
    if meta.shape != shape or not (meta.is_contiguous() and values.is_contiguous()):
        raise ValueError(f"meta must be a contiguous {dtype} tensor of shape {shape}, values contiguous")
    x2, B, o2, out, squeeze = _x_y(x, R, K, out)
    ws, ws_bytes = _workspace(nm_spmv_workspace_bytes(R, K, B), x2, workspace)
    _check(lib.nm_spmv_meta(_ptr(meta), int(fmt), _ptr(values), R, K, _ptr(x2), _ld(x2), B, _ptr(o2), _ld(o2),
                            _ptr(ws), ws_bytes, _stream(x2)))
    return out[0] if squeeze and out.dim() == 2 else out


def nm_spmv_swiglu_workspace_bytes(R: int, K: int, B: int) -> int:
    return int(lib.nm_spmv_swiglu_workspace_bytes(R, K, B))


def dense_gemv_swiglu_workspace_bytes(R: int, K: int, B: int) -> int:
    return int(lib.dense_gemv_swiglu_workspace_bytes(R, K, B))


def nm_spmv_swiglu(gate, up, x: torch.Tensor, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """h = silu(W_gate x) * (W_up x) for packed gate = (masks, values) and up = (masks, values),
    both R x K; x: bf16 [B, K] or [K] -> bf16 [B, R] (or [R])."""
    (gm, gv), (um, uv) = gate, up
    for t, n, dt in ((gm, "gate masks", torch.int32), (gv, "gate values", torch.bfloat16),
                     (um, "up masks", torch.int32), (uv, "up values", torch.bfloat16)):
        _dev(t, n, dt, 2)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    R, K = gm.shape[0], gm.shape[1] * 32
    if gv.shape != (R, K // 2) or um.shape != gm.shape or uv.shape != gv.shape:
        raise ValueError("gate and up must both be packed R x K matrices")
    x2, B, o2, out, squeeze = _x_y(x, R, K, out)
    ws, ws_bytes = _workspace(nm_spmv_swiglu_workspace_bytes(R, K, B), x2, workspace)
    _check(lib.nm_spmv_swiglu(_ptr(gm), _ptr(gv), _ptr(um), _ptr(uv), R, K, _ptr(x2), _ld(x2), B, _ptr(o2),
                              _ld(o2), _ptr(ws), ws_bytes, _stream(x2)))
    return out[0] if squeeze and out.dim() == 2 else out


def dense_gemv_swiglu(W_gate: torch.Tensor, W_up: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Dense baseline of nm_spmv_swiglu: W_gate, W_up bf16 [R, K] with the same row stride."""
    _dev(W_gate, "W_gate", torch.bfloat16, 2)
    _dev(W_up, "W_up", torch.bfloat16, 2)
    if W_gate.shape != W_up.shape or _ld(W_gate) != _ld(W_up):
        raise ValueError("W_gate and W_up must have the same shape and row stride")
    R, K = W_gate.shape
    x2, B, o2, out, squeeze = _x_y(x, R, K, out)
    ws, ws_bytes = _workspace(dense_gemv_swiglu_workspace_bytes(R, K, B), x2, workspace)
    _check(lib.dense_gemv_swiglu(_ptr(W_gate), _ptr(W_up), _ld(W_gate), R, K, _ptr(x2), _ld(x2), B, _ptr(o2),
                                 _ld(o2), _ptr(ws), ws_bytes, _stream(x2)))
    return out[0] if squeeze and out.dim() == 2 else out


def nm_prune_pack_unstructured(W: torch.Tensor, col_norm: torch.Tensor, masks: torch.Tensor | None = None,
                               values: torch.Tensor | None = None):
    """50% unstructured: W bf16 [R, K], col_norm fp32 [K] -> (masks int32 [R, K/32], values bf16 [R, K/2]),
    each row keeping its K/2 highest scores."""
    _dev(W, "W", torch.bfloat16, 2)
    _dev(col_norm, "col_norm", torch.float32, 1)
    R, K = W.shape
    if col_norm.shape[0] != K:
        raise ValueError("col_norm must have K entries")
    if masks is None:
        masks = torch.empty((R, max(K // 32, 1)), dtype=torch.int32, device=W.device)
    if values is None:
        values = torch.empty((R, max(K // 2, 1)), dtype=torch.bfloat16, device=W.device)
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    if not (masks.is_contiguous() and values.is_contiguous()):
        raise ValueError("masks and values must be contiguous")
    if K % 32 == 0 and (masks.shape != (R, K // 32) or values.shape != (R, K // 2)):
        raise ValueError("masks must be [R, K/32] and values [R, K/2]")
    _check(lib.nm_prune_pack_unstructured(_ptr(W), _ld(W), R, K, _ptr(col_norm), _ptr(masks), _ptr(values),
                                          _stream(W)))
    return masks, values


def nm_spmv_unstructured_workspace_bytes(R: int, K: int, B: int) -> int:
    return int(lib.nm_spmv_unstructured_workspace_bytes(R, K, B))


def nm_spmv_unstructured(masks: torch.Tensor, values: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = W_sparse x for 50% unstructured rows packed by nm_prune_pack_unstructured."""
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    if not (masks.is_contiguous() and values.is_contiguous()):
        raise ValueError("masks and values must be contiguous")
    R, K = masks.shape[0], masks.shape[1] * 32
    if values.shape != (R, K // 2):
        raise ValueError("values must be [R, K/2] with K = 32 * masks.shape[1]")
    x2, B, o2, out, squeeze = _x_y(x, R, K, out)
    ws, ws_bytes = _workspace(nm_spmv_unstructured_workspace_bytes(R, K, B), x2, workspace)
    _check(lib.nm_spmv_unstructured(_ptr(masks), _ptr(values), R, K, _ptr(x2), _ld(x2), B, _ptr(o2), _ld(o2),
                                    _ptr(ws), ws_bytes, _stream(x2)))
    return out[0] if squeeze and out.dim() == 2 else out


def nm_unpack_unstructured(masks: torch.Tensor, values: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    R, K = masks.shape[0], masks.shape[1] * 32
    if out is None:
        out = torch.empty((R, K), dtype=torch.bfloat16, device=masks.device)
    _dev(out, "out", torch.bfloat16, 2)
    _check(lib.nm_unpack_unstructured(_ptr(masks), _ptr(values), R, K, _ptr(out), _ld(out), _stream(masks)))
    return out


def nm_hessian(X: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """H = 2 X^T X: X bf16 [T, K] calibration activations -> fp64 [K, K]."""
    _dev(X, "X", torch.bfloat16, 2)
    T, K = X.shape
    if out is None:
        out = torch.empty((K, K), dtype=torch.float64, device=X.device)
    _dev(out, "out", torch.float64, 2)
    if out.shape != (K, K):
        raise ValueError("out must be [K, K]")
    _check(lib.nm_hessian(_ptr(X), T, K, _ld(X), _ptr(out), _ld(out), _stream(X)))
    return out


def nm_obs_inverse_factor_workspace_bytes(K: int) -> int:
    return int(lib.nm_obs_inverse_factor_workspace_bytes(K))


def nm_obs_inverse_factor(H: torch.Tensor, damp: float = 0.01, out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Upper U with U^T U = (H + damp * mean(diag H) * I)^-1 (fp64 [K, K])."""
    _dev(H, "H", torch.float64, 2)
    K = H.shape[0]
    if H.shape != (K, K):
        raise ValueError("H must be square")
    if out is None:
        out = torch.empty((K, K), dtype=torch.float64, device=H.device)
    _dev(out, "out", torch.float64, 2)
    ws, ws_bytes = _workspace(nm_obs_inverse_factor_workspace_bytes(K), H, workspace)
    _check(lib.nm_obs_inverse_factor(_ptr(H), _ld(H), K, float(damp), _ptr(out), _ld(out), _ptr(ws), ws_bytes,
                                     _stream(H)))
    return out


def nm_sparsegpt_workspace_bytes(R: int, K: int) -> int:
    return int(lib.nm_sparsegpt_workspace_bytes(R, K))


def nm_sparsegpt_prune_pack(W: torch.Tensor, H: torch.Tensor, N: int, M: int, damp: float = 0.01,
                            masks: torch.Tensor | None = None, values: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None):
    """OBS / SparseGPT N:M solver: W bf16 [R, K], H fp64 [K, K] -> (masks int32 [R, K/32], values bf16 [R, K/2])."""
    _dev(W, "W", torch.bfloat16, 2)
    _dev(H, "H", torch.float64, 2)
    R, K = W.shape
    if H.shape != (K, K):
        raise ValueError("H must be [K, K]")
    if masks is None:
        masks = torch.empty((R, max(K // 32, 1)), dtype=torch.int32, device=W.device)
    if values is None:
        values = torch.empty((R, max(K // 2, 1)), dtype=torch.bfloat16, device=W.device)
    _dev(masks, "masks", torch.int32, 2)
    _dev(values, "values", torch.bfloat16, 2)
    ws, ws_bytes = _workspace(nm_sparsegpt_workspace_bytes(R, K), W, workspace)
    _check(lib.nm_sparsegpt_prune_pack(_ptr(W), _ld(W), R, K, _ptr(H), _ld(H), int(N), int(M), float(damp),
                                       _ptr(masks), _ptr(values), _ptr(ws), ws_bytes, _stream(W)))
    return masks, values


def _multi_outs(x2, Rs, outs):
    B = x2.shape[0]
    if outs is None:
        outs = [torch.empty((B, R), dtype=torch.bfloat16, device=x2.device) for R in Rs]
    if len(outs) != len(Rs):
        raise ValueError("one output per matrix")
    o2 = []
    for o, R in zip(outs, Rs):
        o = o.unsqueeze(0) if o.dim() == 1 else o
        _dev(o, "out", torch.bfloat16, 2)
        if o.shape != (B, R):
            raise ValueError(f"out must be [{B}, {R}]")
        o2.append(o)
    return outs, o2


def _multi_x(x):
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    _dev(x2, "x", torch.bfloat16, 2)
    return x2


def nm_spmv_multi_workspace_bytes(Rs, K: int, B: int) -> int:
    arr = (_SpmvMatrix * len(Rs))(*[_SpmvMatrix(None, None, int(R), None, int(R)) for R in Rs])
    return int(lib.nm_spmv_multi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(Rs), K, B))


def nm_spmv_multi(packed, x: torch.Tensor, outs=None, workspace: torch.Tensor | None = None):
    """Several packed matrices [(masks, values), ...] sharing x, in one launch -> list of y."""
    x2 = _multi_x(x)
    K = x2.shape[1]
    Rs = []
    for i, (m, v) in enumerate(packed):
        _dev(m, f"masks[{i}]", torch.int32, 2)
        _dev(v, f"values[{i}]", torch.bfloat16, 2)
        if not (m.is_contiguous() and v.is_contiguous()):
            raise ValueError("masks and values must be contiguous")
        if m.shape[1] * 32 != K or v.shape != (m.shape[0], K // 2):
            raise ValueError(f"matrix {i} does not have K={K} columns")
        Rs.append(m.shape[0])
    outs, o2 = _multi_outs(x2, Rs, outs)
    arr = (_SpmvMatrix * len(Rs))(*[_SpmvMatrix(m.data_ptr(), v.data_ptr(), R, o.data_ptr(), _ld(o))
                                     for (m, v), R, o in zip(packed, Rs, o2)])
    ws, ws_bytes = _workspace(int(lib.nm_spmv_multi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(Rs), K,
                                                                     x2.shape[0])), x2, workspace)
    _check(lib.nm_spmv_multi(ctypes.cast(arr, ctypes.c_void_p), len(Rs), K, _ptr(x2), _ld(x2), x2.shape[0], _ptr(ws),
                             ws_bytes, _stream(x2)))
    return outs


def dense_gemv_multi_workspace_bytes(Rs, K: int, B: int) -> int:
    arr = (_DenseMatrix * len(Rs))(*[_DenseMatrix(None, K, int(R), None, int(R)) for R in Rs])
    return int(lib.dense_gemv_multi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(Rs), K, B))


def dense_gemv_multi(Ws, x: torch.Tensor, outs=None, workspace: torch.Tensor | None = None):
    """Several dense matrices sharing x, in one launch -> list of y."""
    x2 = _multi_x(x)
    K = x2.shape[1]
    for i, W in enumerate(Ws):
        _dev(W, f"W[{i}]", torch.bfloat16, 2)
        if W.shape[1] != K:
            raise ValueError(f"matrix {i} does not have K={K} columns")
    Rs = [W.shape[0] for W in Ws]
    outs, o2 = _multi_outs(x2, Rs, outs)
    arr = (_DenseMatrix * len(Rs))(*[_DenseMatrix(W.data_ptr(), _ld(W), R, o.data_ptr(), _ld(o))
                                     for W, R, o in zip(Ws, Rs, o2)])
    ws, ws_bytes = _workspace(int(lib.dense_gemv_multi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(Rs),
                                                                       K, x2.shape[0])), x2, workspace)
    _check(lib.dense_gemv_multi(ctypes.cast(arr, ctypes.c_void_p), len(Rs), K, _ptr(x2), _ld(x2), x2.shape[0],
                                _ptr(ws), ws_bytes, _stream(x2)))
    return outs


def nm_stream_read_sink_words(nbytes: int) -> int:
    return int(lib.nm_stream_read_sink_words(nbytes))


def nm_stream_read(buf: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Measurement aid: one streaming read of a contiguous device tensor (its whole
    storage, a multiple of 16 bytes); returns the per-workgroup XOR folds (int32) whose
    XOR is the XOR of all dwords read."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda":
        raise ValueError("buf must be a tensor on a HIP device")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    words = nm_stream_read_sink_words(nbytes)
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=buf.device)
    _dev(sink, "sink", torch.int32, 1)
    _check(lib.nm_stream_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(buf)))
    return sink


def _plan_dict(pl: _LaunchPlan) -> dict:
    return {f: getattr(pl, f) for f, _ in _LaunchPlan._fields_}


def nm_spmv_plan(R: int, K: int, B: int, epilogue: int = NM_EPI_NONE) -> dict:
    """Launch plan of nm_spmv (or nm_spmv_swiglu with epilogue=NM_EPI_SWIGLU, R rows each)
    on the current device: kernel, threads, grid_x, splits, tiles_per_step,
    x_steps_in_registers, rows_per_group, lds_bytes, workspace_bytes.  Host only."""
    pl = _LaunchPlan()
    _check(lib.nm_spmv_plan(int(R), int(K), int(B), int(epilogue), ctypes.byref(pl)))
    return _plan_dict(pl)


def nm_spmv_multi_plan(rows, K: int, B: int) -> dict:
    """Launch plan of nm_spmv_multi over matrices with the given row counts.  Host only."""
    arr = (ctypes.c_int64 * len(rows))(*[int(r) for r in rows])
    pl = _LaunchPlan()
    _check(lib.nm_spmv_multi_plan(arr, len(rows), int(K), int(B), ctypes.byref(pl)))
    return _plan_dict(pl)
