"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function that include/*.h declares, and rejects invalid arguments synchronously
with the documented status codes before making any HIP call."""
from __future__ import annotations

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# NM_SPMV_LIB: another build of the same ABI (the host-sanitizer run points it at its own)
LIB = os.environ.get("NM_SPMV_LIB") or os.path.join(ROOT, "bitmask_spmv_amd", "libnmspmv.so")

NM_OK, NM_ERR_NULL, NM_ERR_SHAPE, NM_ERR_PATTERN, NM_ERR_ALIGN, NM_ERR_WORKSPACE, NM_ERR_HIP = range(7)


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M):
            name = m.group(1)
            if name not in ("if", "while", "defined"):
                names.add(name)
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB)
    i64, p, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.nm_status_str.argtypes, lib.nm_status_str.restype = [i32], ctypes.c_char_p
    lib.nm_last_error.restype = ctypes.c_char_p
    lib.nm_col_norm.argtypes = [p, i64, i64, i64, p, p]
    lib.nm_prune_pack.argtypes = [p, i64, i64, i64, p, i32, i32, p, p, p]
    lib.nm_spmv.argtypes = [p, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    lib.dense_gemv.argtypes = [p, i64, i64, i64, p, i64, i32, p, i64, p, sz, p]
    lib.nm_unpack.argtypes = [p, p, i64, i64, p, i64, p]
    return lib


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("nm_col_norm", "nm_prune_pack", "nm_spmv", "nm_spmv_workspace_bytes", "dense_gemv",
              "dense_gemv_workspace_bytes", "nm_unpack", "nm_status_str", "nm_last_error", "nm_version",
              "nm_spmv_multi", "nm_spmv_multi_workspace_bytes", "dense_gemv_multi",
              "dense_gemv_multi_workspace_bytes", "nm_meta_from_mask", "nm_spmv_meta", "nm_spmv_swiglu",
              "nm_spmv_swiglu_workspace_bytes", "dense_gemv_swiglu", "dense_gemv_swiglu_workspace_bytes",
              "nm_prune_pack_unstructured", "nm_spmv_unstructured", "nm_spmv_unstructured_workspace_bytes",
              "nm_unpack_unstructured", "nm_hessian", "nm_obs_inverse_factor",
              "nm_obs_inverse_factor_workspace_bytes", "nm_sparsegpt_prune_pack", "nm_sparsegpt_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(L, n)  # resolvable through dlsym


def test_status_strings(L):
    assert L.nm_status_str(0) == b"NM_OK"
    assert L.nm_status_str(3) == b"NM_ERR_PATTERN"
    assert L.nm_status_str(99) == b"NM_ERR_UNKNOWN"
    assert L.nm_version() >= 100


# Fake, never-dereferenced addresses: validation must reject the call before any use.
A16 = 0x10000
A4 = 0x10004
A2 = 0x10002


def test_null_pointers_rejected(L):
    assert L.nm_spmv(None, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_NULL
    assert L.dense_gemv(A16, 64, 4, 64, None, 64, 1, A16, 4, None, 0, None) == NM_ERR_NULL
    assert L.nm_prune_pack(A16, 64, 4, 64, None, 2, 4, A16, A16, None) == NM_ERR_NULL
    assert L.nm_col_norm(None, 16, 64, 64, A16, None) == NM_ERR_NULL
    assert L.nm_unpack(A16, None, 4, 64, A16, 64, None) == NM_ERR_NULL
    assert b"NULL" in L.nm_last_error()


@pytest.mark.parametrize("N,M", [(1, 4), (3, 4), (2, 2), (4, 6), (32, 64), (0, 0), (8, 8)])
def test_patterns_other_than_half_rejected(L, N, M):
    assert L.nm_prune_pack(A16, 64, 4, 64, A16, N, M, A16, A16, None) == NM_ERR_PATTERN


@pytest.mark.parametrize("R,K,B", [(0, 64, 1), (4, 48, 1), (4, 16, 1), (4, 0, 1), (4, 64, 0), (4, 64, 9),
                                   (-1, 64, 1), (1 << 31, 64, 1)])
def test_bad_spmv_shapes_rejected(L, R, K, B):
    assert L.nm_spmv(A4, A16, R, K, A16, max(K, 8), B, A16, max(R, 1), None, 0, None) == NM_ERR_SHAPE


def test_bad_leading_dims_rejected(L):
    assert L.nm_spmv(A4, A16, 4, 64, A16, 32, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE  # ldx < K
    assert L.nm_spmv(A4, A16, 4, 64, A16, 64, 1, A16, 3, None, 0, None) == NM_ERR_SHAPE  # ldy < R
    assert L.dense_gemv(A16, 60, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE  # ldw < K
    assert L.dense_gemv(A16, 64, 4, 60, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE  # K % 8
    assert L.nm_prune_pack(A16, 64, 4, 96, A16, 2, 4, A16, A16, None) == NM_ERR_SHAPE  # ldw < K


def test_misalignment_rejected(L):
    assert L.nm_spmv(A4, A4, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # values
    assert L.nm_spmv(A4, A16, 4, 64, A4, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # x
    assert L.nm_spmv(A4, A16, 4, 64, A16, 68, 2, A16, 4, None, 0, None) == NM_ERR_ALIGN  # ldx % 8
    assert L.nm_spmv(A2, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # masks
    assert L.nm_spmv(A4, A16, 4, 64, A16, 64, 1, 0x10001, 4, None, 0, None) == NM_ERR_ALIGN  # y
    assert L.dense_gemv(A4, 64, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # W
    assert L.dense_gemv(A16, 68, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # ldw
    assert L.nm_prune_pack(A16, 64, 4, 64, A4, 2, 4, A16, A16, None) == NM_ERR_ALIGN  # col_norm
    assert L.nm_unpack(A4, A16, 4, 64, A4, 64, None) == NM_ERR_ALIGN  # W_out


def test_workspace_size_queries_are_consistent(L):
    L.nm_spmv_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    L.nm_spmv_workspace_bytes.restype = ctypes.c_size_t
    L.dense_gemv_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    L.dense_gemv_workspace_bytes.restype = ctypes.c_size_t
    assert L.nm_spmv_workspace_bytes(4, 48, 1) == 0  # invalid shape -> 0
    # split rows need R * B fp32 per slice; a whole-row plan needs nothing
    for R, K, B in [(1024, 4096, 1), (8192, 28672, 8), (4096, 4096, 1)]:
        ws = L.nm_spmv_workspace_bytes(R, K, B)
        assert ws % (4 * R * B) == 0
        ws = L.dense_gemv_workspace_bytes(R, K, B)
        assert ws % (4 * R * B) == 0


class _Mat(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("R", ctypes.c_int64), ("y", ctypes.c_void_p),
                ("ldy", ctypes.c_int64)]


def test_multi_entry_points_reject_bad_arguments(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nm_spmv_multi.argtypes = [p, i32, i64, p, i64, i32, p, sz, p]
    L.dense_gemv_multi.argtypes = [p, i32, i64, p, i64, i32, p, sz, p]
    good = (_Mat * 2)(_Mat(A4, A16, 8, A16, 8), _Mat(A4, A16, 8, A16, 8))
    arr = ctypes.cast(good, ctypes.c_void_p)
    assert L.nm_spmv_multi(None, 2, 64, A16, 64, 1, None, 0, None) == NM_ERR_NULL
    assert L.nm_spmv_multi(arr, 2, 64, None, 64, 1, None, 0, None) == NM_ERR_NULL
    assert L.nm_spmv_multi(arr, 0, 64, A16, 64, 1, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_multi(arr, 9, 64, A16, 64, 1, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_multi(arr, 2, 48, A16, 64, 1, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_multi(arr, 2, 64, A16, 64, 9, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_multi(arr, 2, 64, A4, 64, 1, None, 0, None) == NM_ERR_ALIGN
    bad = (_Mat * 2)(_Mat(A4, A16, 8, A16, 8), _Mat(A4, None, 8, A16, 8))
    assert L.nm_spmv_multi(ctypes.cast(bad, p), 2, 64, A16, 64, 1, None, 0, None) == NM_ERR_NULL
    bad = (_Mat * 2)(_Mat(A4, A16, 8, A16, 8), _Mat(A4, A4, 8, A16, 8))
    assert L.nm_spmv_multi(ctypes.cast(bad, p), 2, 64, A16, 64, 1, None, 0, None) == NM_ERR_ALIGN
    bad = (_Mat * 2)(_Mat(A4, A16, 8, A16, 8), _Mat(A4, A16, 0, A16, 8))
    assert L.nm_spmv_multi(ctypes.cast(bad, p), 2, 64, A16, 64, 1, None, 0, None) == NM_ERR_SHAPE
    dgood = (_Mat * 1)(_Mat(A16, 64, 8, A16, 8))
    assert L.dense_gemv_multi(ctypes.cast(dgood, p), 1, 64, None, 64, 1, None, 0, None) == NM_ERR_NULL
    assert L.dense_gemv_multi(ctypes.cast(dgood, p), 1, 60, A16, 64, 1, None, 0, None) == NM_ERR_SHAPE
    dbad = (_Mat * 1)(_Mat(A4, 64, 8, A16, 8))
    assert L.dense_gemv_multi(ctypes.cast(dbad, p), 1, 64, A16, 64, 1, None, 0, None) == NM_ERR_ALIGN


def test_metadata_entry_points_reject_bad_arguments(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nm_meta_from_mask.argtypes = [p, i64, i64, i32, p, p]
    L.nm_spmv_meta.argtypes = [p, i32, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    # conversion
    assert L.nm_meta_from_mask(None, 4, 64, 1, A16, None) == NM_ERR_NULL
    assert L.nm_meta_from_mask(A4, 4, 64, 1, None, None) == NM_ERR_NULL
    assert L.nm_meta_from_mask(A4, 4, 64, 0, A16, None) == NM_ERR_PATTERN  # bitmask: nothing to convert
    assert L.nm_meta_from_mask(A4, 4, 64, 3, A16, None) == NM_ERR_PATTERN
    assert L.nm_meta_from_mask(A4, 4, 48, 1, A16, None) == NM_ERR_SHAPE
    assert L.nm_meta_from_mask(A4, 0, 64, 2, A16, None) == NM_ERR_SHAPE
    assert L.nm_meta_from_mask(A2, 4, 64, 2, A16, None) == NM_ERR_ALIGN
    assert L.nm_meta_from_mask(A4, 4, 64, 2, A4, None) == NM_ERR_ALIGN
    # product
    assert L.nm_spmv_meta(None, 1, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_NULL
    assert L.nm_spmv_meta(A16, 7, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_PATTERN
    assert L.nm_spmv_meta(A16, -1, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_PATTERN
    assert L.nm_spmv_meta(A16, 1, A16, 4, 48, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_meta(A16, 2, A16, 4, 64, A16, 64, 9, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_meta(A4, 1, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # u8 meta
    assert L.nm_spmv_meta(A4, 2, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # i32 meta
    assert L.nm_spmv_meta(A2, 0, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # masks
    assert L.nm_spmv_meta(A16, 1, A4, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN  # values


def test_swiglu_entry_points_reject_bad_arguments(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nm_spmv_swiglu.argtypes = [p, p, p, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.dense_gemv_swiglu.argtypes = [p, p, i64, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.nm_spmv_swiglu_workspace_bytes.argtypes = [i64, i64, i32]
    L.nm_spmv_swiglu_workspace_bytes.restype = sz
    assert L.nm_spmv_swiglu(A4, A16, None, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_NULL
    assert L.nm_spmv_swiglu(A4, A16, A4, A16, 4, 48, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_swiglu(A4, A16, A4, A16, 1 << 29 + 1, 64, A16, 64, 1, A16, 1 << 30, None, 0, None) \
        == NM_ERR_SHAPE
    assert L.nm_spmv_swiglu(A4, A16, A4, A16, 4, 64, A16, 64, 0, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_swiglu(A4, A16, A4, A4, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN
    assert L.nm_spmv_swiglu(A4, A16, A2, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN
    assert L.dense_gemv_swiglu(A16, None, 64, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_NULL
    assert L.dense_gemv_swiglu(A16, A16, 60, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.dense_gemv_swiglu(A16, A4, 64, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN
    assert L.nm_spmv_swiglu_workspace_bytes(0, 64, 1) == 0
    assert L.nm_spmv_swiglu_workspace_bytes(8, 8192, 1) % (4 * 16) == 0


def test_unstructured_entry_points_reject_bad_arguments(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nm_prune_pack_unstructured.argtypes = [p, i64, i64, i64, p, p, p, p]
    L.nm_spmv_unstructured.argtypes = [p, p, i64, i64, p, i64, i32, p, i64, p, sz, p]
    L.nm_unpack_unstructured.argtypes = [p, p, i64, i64, p, i64, p]
    L.nm_spmv_unstructured_workspace_bytes.argtypes = [i64, i64, i32]
    L.nm_spmv_unstructured_workspace_bytes.restype = sz
    assert L.nm_prune_pack_unstructured(A16, 64, 4, 64, None, A16, A16, None) == NM_ERR_NULL
    assert L.nm_prune_pack_unstructured(A16, 64, 4, 48, A16, A16, A16, None) == NM_ERR_SHAPE
    assert L.nm_prune_pack_unstructured(A16, 60, 4, 64, A16, A16, A16, None) == NM_ERR_SHAPE
    assert L.nm_prune_pack_unstructured(A4, 64, 4, 64, A16, A16, A16, None) == NM_ERR_ALIGN
    assert L.nm_prune_pack_unstructured(A16, 64, 4, 64, A4, A16, A16, None) == NM_ERR_ALIGN
    assert L.nm_spmv_unstructured(None, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_NULL
    assert L.nm_spmv_unstructured(A4, A16, 4, 48, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_unstructured(A4, A16, 0, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_unstructured(A4, A16, 4, 64, A16, 64, 9, A16, 4, None, 0, None) == NM_ERR_SHAPE
    assert L.nm_spmv_unstructured(A4, A4, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN
    assert L.nm_spmv_unstructured(A2, A16, 4, 64, A16, 64, 1, A16, 4, None, 0, None) == NM_ERR_ALIGN
    assert L.nm_unpack_unstructured(A4, A16, 4, 64, None, 64, None) == NM_ERR_NULL
    assert L.nm_unpack_unstructured(A4, A16, 4, 64, A4, 64, None) == NM_ERR_ALIGN
    assert L.nm_spmv_unstructured_workspace_bytes(4, 48, 1) == 0
    assert L.nm_spmv_unstructured_workspace_bytes(16, 8192, 2) % (4 * 16 * 2) == 0


def test_solver_entry_points_reject_bad_arguments(L):
    p, i64, i32, sz, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    L.nm_hessian.argtypes = [p, i64, i64, i64, p, i64, p]
    L.nm_obs_inverse_factor.argtypes = [p, i64, i64, f64, p, i64, p, sz, p]
    L.nm_obs_inverse_factor_workspace_bytes.argtypes = [i64]
    L.nm_obs_inverse_factor_workspace_bytes.restype = sz
    L.nm_sparsegpt_workspace_bytes.argtypes = [i64, i64]
    L.nm_sparsegpt_workspace_bytes.restype = sz
    L.nm_sparsegpt_prune_pack.argtypes = [p, i64, i64, i64, p, i64, i32, i32, f64, p, p, p, sz, p]
    assert L.nm_hessian(None, 4, 64, 64, A16, 64, None) == NM_ERR_NULL
    assert L.nm_hessian(A16, 0, 64, 64, A16, 64, None) == NM_ERR_SHAPE
    assert L.nm_hessian(A16, 4, 64, 32, A16, 64, None) == NM_ERR_SHAPE
    assert L.nm_hessian(A16, 4, 64, 64, A16, 63, None) == NM_ERR_SHAPE
    assert L.nm_hessian(A16, 4, 64, 64, A4, 64, None) == NM_ERR_ALIGN
    assert L.nm_obs_inverse_factor_workspace_bytes(48) == 0
    wsb = L.nm_obs_inverse_factor_workspace_bytes(64)
    assert wsb >= 2 * 64 * 64 * 8
    assert L.nm_obs_inverse_factor(A16, 64, 48, 0.01, A16, 64, A16, wsb, None) == NM_ERR_SHAPE
    assert L.nm_obs_inverse_factor(A16, 64, 64, -1.0, A16, 64, A16, wsb, None) == NM_ERR_SHAPE
    assert L.nm_obs_inverse_factor(A16, 64, 64, float("nan"), A16, 64, A16, wsb, None) == NM_ERR_SHAPE
    assert L.nm_obs_inverse_factor(A16, 64, 64, 0.01, None, 64, A16, wsb, None) == NM_ERR_NULL
    assert L.nm_obs_inverse_factor(A16, 64, 64, 0.01, A16, 64, A16, wsb - 8, None) == NM_ERR_WORKSPACE
    assert L.nm_obs_inverse_factor(A4, 64, 64, 0.01, A16, 64, A16, wsb, None) == NM_ERR_ALIGN
    swb = L.nm_sparsegpt_workspace_bytes(8, 64)
    assert swb >= wsb + 8 * 64 * 8
    assert L.nm_sparsegpt_prune_pack(A16, 64, 8, 64, A16, 64, 3, 4, 0.01, A16, A16, A16, swb, None) == NM_ERR_PATTERN
    assert L.nm_sparsegpt_prune_pack(A16, 64, 8, 48, A16, 64, 2, 4, 0.01, A16, A16, A16, swb, None) == NM_ERR_SHAPE
    assert L.nm_sparsegpt_prune_pack(A16, 64, 8, 64, A16, 64, 2, 4, 0.01, A16, A4, A16, swb, None) == NM_ERR_ALIGN
    assert L.nm_sparsegpt_prune_pack(A16, 64, 8, 64, A16, 64, 2, 4, 0.01, A16, A16, None, 0, None) == NM_ERR_WORKSPACE
    assert L.nm_sparsegpt_prune_pack(None, 64, 8, 64, A16, 64, 2, 4, 0.01, A16, A16, A16, swb, None) == NM_ERR_NULL


def test_stream_read_rejects_bad_arguments(L):
    p, sz = ctypes.c_void_p, ctypes.c_size_t
    L.nm_stream_read_sink_words.argtypes, L.nm_stream_read_sink_words.restype = [sz], sz
    L.nm_stream_read.argtypes, L.nm_stream_read.restype = [p, sz, p, sz, p], ctypes.c_int
    # one fold per wave: 8 per 512-thread workgroup, at most 1024 workgroups, and at least
    # one 2 KiB unit per wave (16 KiB per workgroup)
    assert L.nm_stream_read_sink_words(16) == 8
    assert L.nm_stream_read_sink_words(1 << 31) == 256 * 8  # one 8-wave workgroup per CU of 256
    assert L.nm_stream_read_sink_words(16384 * 3) == 3 * 8  # two 1 KiB units per wave at least
    assert L.nm_stream_read_sink_words(16384 * 3 + 16) == 3 * 8
    assert L.nm_stream_read_sink_words(16384 * 4) == 4 * 8
    words = L.nm_stream_read_sink_words(1 << 20)
    assert L.nm_stream_read(None, 1 << 20, A16, words, None) == NM_ERR_NULL
    assert L.nm_stream_read(A16, 1 << 20, None, words, None) == NM_ERR_NULL
    assert L.nm_stream_read(A16, 0, A16, words, None) == NM_ERR_SHAPE
    assert L.nm_stream_read(A16, 24, A16, words, None) == NM_ERR_SHAPE
    assert L.nm_stream_read(A16, (1 << 31) + 16, A16, 1024, None) == NM_ERR_SHAPE
    assert L.nm_stream_read(A4, 1 << 20, A16, words, None) == NM_ERR_ALIGN
    assert L.nm_stream_read(A16, 1 << 20, A16, words - 1, None) == NM_ERR_WORKSPACE


def test_noalloc_rejects_bad_arguments_and_oversized_scratch(L):
    """nm_spmv_noalloc validates like nm_spmv and rejects, before any HIP call, a shape whose
    split-row partial sums exceed its fixed 4 MiB scratch (B = 2, K = 28672 splits every row
    in two: 2 * 2 * R * 4 bytes)."""
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.nm_spmv_noalloc.argtypes = [p, p, i64, i64, p, i64, i32, p, i64, p]
    L.nm_spmv_noalloc.restype = i32
    assert L.nm_spmv_noalloc(None, A16, 4, 64, A16, 64, 1, A16, 4, None) == NM_ERR_NULL
    assert L.nm_spmv_noalloc(A4, A16, 4, 48, A16, 64, 1, A16, 4, None) == NM_ERR_SHAPE
    assert L.nm_spmv_noalloc(A4, A16, 4, 64, A16, 64, 9, A16, 4, None) == NM_ERR_SHAPE
    assert L.nm_spmv_noalloc(A4, A4, 4, 64, A16, 64, 1, A16, 4, None) == NM_ERR_ALIGN
    K = 28672
    assert L.nm_spmv_noalloc(A4, A16, 300000, K, A16, K, 2, A16, 300000, None) == NM_ERR_WORKSPACE
    assert b"scratch" in L.nm_last_error()
    # exactly at the limit (262144 rows: 4 MiB) the shape is accepted; without a GPU the
    # call then fails at the device lookup, not at the size check
    assert L.nm_spmv_noalloc(A4, A16, 262144, K, A16, K, 2, A16, 262144, None) not in (NM_ERR_WORKSPACE, NM_OK)


class _Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("threads", ctypes.c_int), ("grid_x", ctypes.c_int),
                ("splits", ctypes.c_int), ("tiles_per_step", ctypes.c_int), ("x_steps_in_registers", ctypes.c_int),
                ("rows_per_group", ctypes.c_int), ("lds_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]


def test_launch_plans_host_only(L):
    """nm_spmv_plan / nm_spmv_multi_plan run the planners on the host (256 compute units
    assumed without a GPU): word-per-lane walk at 1-2 tokens (whole rows, half rows or
    strips per wave at one token), matrix-core tiles at 8, x kept in registers where each
    wave has exactly four steps per unit, workspace only with split rows; invalid sizes, a
    NULL plan and an unknown epilogue are rejected."""
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.nm_spmv_plan.argtypes, L.nm_spmv_plan.restype = [i64, i64, i32, i32, p], i32
    L.nm_spmv_multi_plan.argtypes, L.nm_spmv_multi_plan.restype = [p, i32, i64, i32, p], i32
    pl = _Plan()
    for R, K in [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (8192, 8192), (28672, 8192),
                 (8192, 28672), (5120, 17408), (5121, 25600), (1, 32), (3, 28672)]:
        for B in (1, 2, 4, 8):
            for epi in (0, 1):
                assert L.nm_spmv_plan(R, K, B, epi, ctypes.byref(pl)) == NM_OK, (R, K, B, epi)
                assert pl.threads in (256, 512, 1024) and pl.grid_x >= 1 and pl.splits >= 1
                assert (pl.workspace_bytes > 0) == (pl.splits > 1)
                if pl.kernel == 1:
                    assert pl.splits == 1 and pl.tiles_per_step in (1, 2) and pl.lds_bytes == 0
                    assert pl.x_steps_in_registers in (0, 4)
                else:
                    assert pl.tiles_per_step == 0 and pl.x_steps_in_registers == 0 and pl.lds_bytes > 0
                if pl.kernel in (2, 3):  # half rows / strips: one matrix, one token, no split
                    assert B == 1 and epi == 0 and pl.splits == 1 and pl.threads in (512, 1024)
                if pl.kernel == 3:  # every row in exactly one workgroup
                    assert pl.rows_per_group >= 1 and (pl.grid_x - 1) * pl.rows_per_group < R <= pl.grid_x * pl.rows_per_group
                else:
                    assert pl.rows_per_group == 0
                if B <= 2:
                    assert pl.kernel in (0, 2, 3)
    assert L.nm_spmv_plan(14336, 4096, 8, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.threads, pl.x_steps_in_registers) == (1, 512, 4)
    assert L.nm_spmv_plan(28672, 8192, 8, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.threads, pl.x_steps_in_registers) == (1, 1024, 4)
    assert L.nm_spmv_plan(8192, 28672, 8, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.tiles_per_step, pl.x_steps_in_registers) == (1, 2, 0)
    assert L.nm_spmv_plan(4096, 14336, 1, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.threads, pl.grid_x) == (2, 1024, 512)
    assert L.nm_spmv_plan(4096, 14336, 2, 0, ctypes.byref(pl)) == NM_OK and pl.kernel == 0
    assert L.nm_spmv_plan(8192, 28672, 1, 0, ctypes.byref(pl)) == NM_OK and (pl.kernel, pl.grid_x) == (2, 1024)
    # 5120 rows of 7+ strips: strips of 10 rows per 16-wave workgroup, one workgroup round
    assert L.nm_spmv_plan(5120, 17408, 1, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.threads, pl.grid_x, pl.rows_per_group) == (3, 1024, 512, 10)
    assert L.nm_spmv_plan(5121, 17408, 1, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.grid_x, pl.rows_per_group) == (3, 466, 11)
    # rows of 8192 columns: strips of consecutive rows per 8-wave workgroup
    assert L.nm_spmv_plan(8192, 8192, 1, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.threads, pl.grid_x, pl.rows_per_group) == (3, 512, 1024, 8)
    assert L.nm_spmv_plan(28672, 8192, 1, 0, ctypes.byref(pl)) == NM_OK
    assert (pl.kernel, pl.threads, pl.rows_per_group) == (3, 512, 28)
    for R, K in [(14336, 4096), (4096, 4096), (1024, 8192), (6000, 8192), (17408, 5120)]:  # whole rows
        assert L.nm_spmv_plan(R, K, 1, 0, ctypes.byref(pl)) == NM_OK and pl.kernel == 0, (R, K)
    assert L.nm_spmv_plan(8192, 8192, 2, 0, ctypes.byref(pl)) == NM_OK and pl.kernel == 0
    assert L.nm_spmv_plan(8192, 8192, 1, 1, ctypes.byref(pl)) == NM_OK and pl.kernel == 0
    assert L.nm_spmv_plan(4096, 14336, 1, 1, ctypes.byref(pl)) == NM_OK and pl.kernel == 0  # gated MLP
    rows = (ctypes.c_int64 * 3)(4096, 1024, 1024)
    assert L.nm_spmv_multi_plan(rows, 3, 4096, 1, ctypes.byref(pl)) == NM_OK and pl.kernel == 0
    assert L.nm_spmv_multi_plan(rows, 3, 4096, 8, ctypes.byref(pl)) == NM_OK and pl.kernel == 1
    assert L.nm_spmv_plan(4096, 4096, 1, 0, None) == NM_ERR_NULL
    assert L.nm_spmv_plan(4096, 4096, 1, 2, ctypes.byref(pl)) == NM_ERR_PATTERN
    for R, K, B in [(0, 64, 1), (4, 48, 1), (4, 64, 0), (4, 64, 9), (1 << 31, 64, 1)]:
        assert L.nm_spmv_plan(R, K, B, 0, ctypes.byref(pl)) == NM_ERR_SHAPE
    assert L.nm_spmv_multi_plan(None, 3, 4096, 1, ctypes.byref(pl)) == NM_ERR_NULL
    assert L.nm_spmv_multi_plan(rows, 0, 4096, 1, ctypes.byref(pl)) == NM_ERR_SHAPE
    assert L.nm_spmv_multi_plan(rows, 9, 4096, 1, ctypes.byref(pl)) == NM_ERR_SHAPE


C_CLIENT = r"""
#include "nm_spmv.h"
#include <stdio.h>

int main(void) {
    nm_launch_plan plan;
    const nm_status s = nm_spmv_plan(4096, 14336, 1, NM_EPI_NONE, &plan);
    if (s != NM_OK) { printf("plan: %s\n", nm_status_str(s)); return 1; }
    /* argument errors come back synchronously, before any HIP call */
    if (nm_spmv(NULL, NULL, 4096, 14336, NULL, 14336, 1, NULL, 4096, NULL, 0, NULL) != NM_ERR_NULL) return 2;
    if (nm_last_error()[0] == '\0') return 3;
    printf("version %d kernel %d threads %d grid %d\n", nm_version(), plan.kernel, plan.threads, plan.grid_x);
    return 0;
}
"""


def test_plain_c_client_builds_and_runs(tmp_path):
    """The header is plain C (C99, no C++ or HIP types): a C program includes it, links the
    library and calls the host-only entry points; the header also compiles as C++."""
    if os.environ.get("NM_SPMV_LIB"):
        pytest.skip("the C client links the regular build (a sanitized one needs its runtimes)")
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(LIB)
    cc = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
          str(src), "-o", str(exe), f"-L{libdir}", f"-l:{os.path.basename(LIB)}", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert re.match(r"version \d+ kernel 2 threads 1024 grid 512", r.stdout), r.stdout
    cxx = tmp_path / "client.cpp"
    cxx.write_text('#include "nm_spmv.h"\nint main() { return nm_version() > 0 ? 0 : 1; }\n')
    r = subprocess.run(["g++", "-std=c++11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        f"-I{os.path.join(ROOT, 'include')}", str(cxx)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
