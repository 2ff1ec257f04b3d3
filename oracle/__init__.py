"""CPU oracle for the N:M bitmask decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product library (``bitmask_spmv_amd``) never
imports it, and it never imports the product library: the two share no code.

The arithmetic lives in ``nm_oracle.c`` (plain C, IEEE fp64, built with
``-ffp-contract=off``); this module only marshals numpy arrays to it.  The function
list and the passages each follows:

* ``col_norm``   -- Wanda activation norm n_j = sqrt(sum_t X[t][j]^2)
                    ("SparseDecoding：只用解码激活校准的稀疏推理", 核心公式)
* ``prune_pack`` -- score |W_ij| * n_j, keep the top N of every M columns (ties to
                    the lower column), one uint32 mask word per 32 columns (bit b <->
                    column 32w+b), kept values in increasing column order
                    ("SparseDecoding: Decoding-Aware Pruning ...", Methodology Steps 2-3;
                    "SparseDecoding:解码感知的准确高效大模型剪枝框架", 前置知识 N:M, 方法步骤详情 第三步)
* ``unpack``     -- inverse of the packing: dense pruned matrix, zeros elsewhere
* ``spmv``       -- fp64 matvec of the unpacked pruned matrix (+ sum of |products|)
* ``dense``      -- fp64 matvec of the dense matrix (+ sum of |products|)
* ``meta_from_mask`` / ``spmv_index`` -- the index formats the bitmask is priced
                    against (uint8 offset within the 32-column word, int32 column index
                    within the row, one per kept weight in value order) and the fp64
                    matvec defined directly over them
                    ("SparseDecoding: Decoding-Aware Pruning ...", Main Findings;
                    "SparseDecoding:解码感知的准确高效大模型剪枝框架", 核心方法 核心创新二)

* ``prune_pack_unstructured`` / ``unpack_unstructured`` / ``spmv_unstructured`` -- the
                    pages' 50% unstructured setting: each row keeps its K/2 highest scores
                    (same score and tie rule), same bitmask + ascending-values encoding
                    with a varying number of set bits per word
                    ("SparseDecoding: Decoding-Aware Pruning ...", Methodology Steps 3-4)
* ``swiglu`` / ``swiglu_tolerance`` -- h = silu(g) * u, silu(g) = g / (1 + exp(-g)), on
                    fp64 gate and up products (the gated MLP of the models the pages
                    evaluate: Llama-3.1-8B, Llama-3.3-70B, Qwen3), and the error bound a
                    result inherits from the matvec tolerance of g and u

The OBS / SparseGPT N:M solver oracle (Hessian, inverse factor, column-sequential
selection and compensation) lives in ``oracle/sparsegpt.py`` (plain numpy, fp64).

Pins (tests that tie the oracle to something other than itself) live in
``tests/test_oracle_pins.py``; every function above has at least one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nm_oracle.c")
_LIB = os.path.join(_HERE, "libnmoracle.so")
# NM_ORACLE_LIB: another build of nm_oracle.c to load (the host-sanitizer run points it
# at an instrumented one); build() always writes _LIB
_LOAD = os.environ.get("NM_ORACLE_LIB") or _LIB

_lib = None


class OracleError(RuntimeError):
    pass


_ERRS = {1: "bad argument", 2: "non-finite input", 3: "mask word without exactly 16 set bits (or malformed index metadata)",
         4: "out of memory"}


def build(force: bool = True) -> str:
    """Compile nm_oracle.c into a host-only shared library next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LOAD == _LIB and not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LOAD)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.nmo_col_norm.argtypes = [p, i64, i64, i64, p]
    lib.nmo_prune_pack.argtypes = [p, i64, i64, i64, p, ctypes.c_int, ctypes.c_int, p, p]
    lib.nmo_unpack.argtypes = [p, p, i64, i64, p]
    lib.nmo_spmv.argtypes = [p, p, i64, i64, p, i64, ctypes.c_int, p, p, ctypes.c_int]
    lib.nmo_dense.argtypes = [p, i64, i64, i64, p, i64, ctypes.c_int, p, p, ctypes.c_int]
    lib.nmo_meta_from_mask.argtypes = [p, i64, i64, ctypes.c_int, p]
    lib.nmo_prune_pack_unstructured.argtypes = [p, i64, i64, i64, p, p, p]
    lib.nmo_unpack_unstructured.argtypes = [p, p, i64, i64, p]
    lib.nmo_spmv_unstructured.argtypes = [p, p, i64, i64, p, i64, ctypes.c_int, p, p, ctypes.c_int]
    lib.nmo_spmv_index.argtypes = [p, ctypes.c_int, p, i64, i64, p, i64, ctypes.c_int, p, p, ctypes.c_int]
    for f in (lib.nmo_col_norm, lib.nmo_prune_pack, lib.nmo_unpack, lib.nmo_spmv, lib.nmo_dense,
              lib.nmo_meta_from_mask, lib.nmo_spmv_index, lib.nmo_prune_pack_unstructured,
              lib.nmo_unpack_unstructured, lib.nmo_spmv_unstructured):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {_ERRS.get(rc, rc)}")


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected raw bfloat16 patterns as uint16")
    return a


def col_norm(X) -> np.ndarray:
    """X: uint16 bf16 patterns [T, K] -> float32 [K]."""
    X = _u16(X)
    T, K = X.shape
    n = np.empty(K, dtype=np.float32)
    _check(_load().nmo_col_norm(_ptr(X), T, K, K, _ptr(n)), "col_norm")
    return n


def prune_pack(W, n, N: int, M: int):
    """W: uint16 [R, K]; n: float32 [K] -> (masks uint32 [R, K/32], values uint16 [R, K/2])."""
    W = _u16(W)
    n = np.ascontiguousarray(n, dtype=np.float32)
    R, K = W.shape
    if n.shape != (K,):
        raise ValueError("col_norm length must equal K")
    if K % 32:
        raise OracleError("prune_pack: bad argument")
    masks = np.empty((R, K // 32), dtype=np.uint32)
    values = np.empty((R, K // 2), dtype=np.uint16)
    _check(_load().nmo_prune_pack(_ptr(W), K, R, K, _ptr(n), int(N), int(M), _ptr(masks), _ptr(values)),
           "prune_pack")
    return masks, values


def unpack(masks, values, K: int) -> np.ndarray:
    masks = np.ascontiguousarray(masks, dtype=np.uint32)
    values = _u16(values)
    R = masks.shape[0]
    out = np.empty((R, K), dtype=np.uint16)
    _check(_load().nmo_unpack(_ptr(masks), _ptr(values), R, K, _ptr(out)), "unpack")
    return out


def spmv(masks, values, x, K: int, nthreads: int = 1):
    """-> (y fp64 [B, R], absum fp64 [B, R]) for the packed pruned matrix."""
    masks = np.ascontiguousarray(masks, dtype=np.uint32)
    values = _u16(values)
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    R = masks.shape[0]
    B = x.shape[0]
    if x.shape[1] != K or masks.shape != (R, K // 32) or values.shape != (R, K // 2):
        raise ValueError("shape mismatch")
    y = np.empty((B, R), dtype=np.float64)
    a = np.empty((B, R), dtype=np.float64)
    _check(_load().nmo_spmv(_ptr(masks), _ptr(values), R, K, _ptr(x), K, B, _ptr(y), _ptr(a), int(nthreads)),
           "spmv")
    return y, a


def dense(W, x, nthreads: int = 1):
    """-> (y fp64 [B, R], absum fp64 [B, R]) for the dense matrix."""
    W = _u16(W)
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    R, K = W.shape
    B = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("shape mismatch")
    y = np.empty((B, R), dtype=np.float64)
    a = np.empty((B, R), dtype=np.float64)
    _check(_load().nmo_dense(_ptr(W), K, R, K, _ptr(x), K, B, _ptr(y), _ptr(a), int(nthreads)), "dense")
    return y, a


def prune_pack_unstructured(W, n):
    """W: uint16 [R, K]; n: float32 [K] -> (masks uint32 [R, K/32], values uint16 [R, K/2]), K/2 kept per row."""
    W = _u16(W)
    n = np.ascontiguousarray(n, dtype=np.float32)
    R, K = W.shape
    if n.shape != (K,):
        raise ValueError("col_norm length must equal K")
    if K % 32:
        raise OracleError("prune_pack_unstructured: bad argument")
    masks = np.empty((R, K // 32), dtype=np.uint32)
    values = np.empty((R, K // 2), dtype=np.uint16)
    _check(_load().nmo_prune_pack_unstructured(_ptr(W), K, R, K, _ptr(n), _ptr(masks), _ptr(values)),
           "prune_pack_unstructured")
    return masks, values


def unpack_unstructured(masks, values, K: int) -> np.ndarray:
    masks = np.ascontiguousarray(masks, dtype=np.uint32)
    values = _u16(values)
    R = masks.shape[0]
    out = np.empty((R, K), dtype=np.uint16)
    _check(_load().nmo_unpack_unstructured(_ptr(masks), _ptr(values), R, K, _ptr(out)), "unpack_unstructured")
    return out


def spmv_unstructured(masks, values, x, K: int, nthreads: int = 1):
    """-> (y fp64 [B, R], absum fp64 [B, R]) for unstructured rows (K/2 set bits per row)."""
    masks = np.ascontiguousarray(masks, dtype=np.uint32)
    values = _u16(values)
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    R = masks.shape[0]
    B = x.shape[0]
    if x.shape[1] != K or masks.shape != (R, K // 32) or values.shape != (R, K // 2):
        raise ValueError("shape mismatch")
    y = np.empty((B, R), dtype=np.float64)
    a = np.empty((B, R), dtype=np.float64)
    _check(_load().nmo_spmv_unstructured(_ptr(masks), _ptr(values), R, K, _ptr(x), K, B, _ptr(y), _ptr(a),
                                         int(nthreads)), "spmv_unstructured")
    return y, a


META_U8, META_I32 = 1, 2
_META_DT = {META_U8: np.uint8, META_I32: np.int32}


def meta_from_mask(masks, K: int, fmt: int) -> np.ndarray:
    """masks uint32 [R, K/32] -> uint8 [R, K/2] offsets (META_U8) or int32 [R, K/2] indices (META_I32)."""
    masks = np.ascontiguousarray(masks, dtype=np.uint32)
    if fmt not in _META_DT:
        raise OracleError("meta_from_mask: bad argument")
    R = masks.shape[0]
    out = np.empty((R, K // 2), dtype=_META_DT[fmt])
    _check(_load().nmo_meta_from_mask(_ptr(masks), R, K, int(fmt), _ptr(out)), "meta_from_mask")
    return out


def spmv_index(meta, fmt: int, values, x, K: int, nthreads: int = 1):
    """-> (y fp64 [B, R], absum fp64 [B, R]) with the kept weights placed by index metadata."""
    if fmt not in _META_DT:
        raise OracleError("spmv_index: bad argument")
    meta = np.ascontiguousarray(meta, dtype=_META_DT[fmt])
    values = _u16(values)
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    R = values.shape[0]
    B = x.shape[0]
    if x.shape[1] != K or meta.shape != (R, K // 2) or values.shape != (R, K // 2):
        raise ValueError("shape mismatch")
    y = np.empty((B, R), dtype=np.float64)
    a = np.empty((B, R), dtype=np.float64)
    _check(_load().nmo_spmv_index(_ptr(meta), int(fmt), _ptr(values), R, K, _ptr(x), K, B, _ptr(y), _ptr(a),
                                  int(nthreads)), "spmv_index")
    return y, a


def swiglu(g, u) -> np.ndarray:
    """fp64 h = silu(g) * u with silu(g) = g / (1 + exp(-g))."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


SILU_SLOPE_BOUND = 1.1  # sup |d silu / dg| = 1.0998... (pinned in the tests)


def swiglu_tolerance(g, ag, u, au, rel: float = 1e-2, abs_frac: float = 1e-3) -> np.ndarray:
    """Bound on |h_test - h_ref| when g and u each meet the matvec tolerance
    e = rel*|ref| + abs_frac*sum|products| and h is rounded once to bf16:
    |silu(g')u' - silu(g)u| <= L*eg*(|u| + eu) + |silu(g)|*eu, L = SILU_SLOPE_BOUND,
    plus half-ulp-of-bf16 relative rounding (2^-8) on top of the result's magnitude."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    eg = rel * np.abs(g) + abs_frac * np.asarray(ag, dtype=np.float64)
    eu = rel * np.abs(u) + abs_frac * np.asarray(au, dtype=np.float64)
    with np.errstate(over="ignore"):
        sg = np.abs(g / (1.0 + np.exp(-g)))
    pre = SILU_SLOPE_BOUND * eg * (np.abs(u) + eu) + sg * eu
    return pre + 2.0 ** -8 * (sg * np.abs(u) + pre) + 1e-30


def within_tolerance(y_test, y_ref, absum, rel: float = 1e-2, abs_frac: float = 1e-3) -> np.ndarray:
    """Element-wise acceptance |y - y_ref| <= rel*|y_ref| + abs_frac*sum_j|W_ij x_j|."""
    y_test = np.asarray(y_test, dtype=np.float64)
    return np.abs(y_test - y_ref) <= rel * np.abs(y_ref) + abs_frac * absum
