"""fp64 CPU oracle of the SNACK COO layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``coo_spmm_row_amd``)
never imports it, and it imports nothing from the product.

The arithmetic lives in ``snack_oracle.c`` (plain C, fp64, optional OpenMP
over independent outputs).  This module compiles it with gcc, loads it with
ctypes and converts numpy inputs: fp32 values are widened to fp64 exactly, bf16
inputs are given as their exact fp32 images.

Source: "Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks on
GPU" (arXiv:2610.04093): Algorithm 1 (forward), Section 3.4 and Appendix F
(both gradients), Appendix B Table 7 (COO/CSR/CSC), Algorithm 2 and Appendix G
(prune-and-regrow topology update).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "snack_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ERRORS = {0: "ok", 1: "null", 2: "shape", 3: "index", 4: "duplicate", 5: "nomem"}


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed: {ERRORS.get(code, code)}")
        self.code = code
        self.kind = ERRORS.get(code, str(code))


def build(force: bool = True) -> str:
    """Compile snack_oracle.c into liboracle.so next to it (gcc -O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def configure(lib):
    """Declare the C signatures on a loaded liboracle."""
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_build.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p, p, p, p, p]
    lib.oracle_fwd.argtypes = [i64, i64, i64, p, p, p, i64, p, p, p, ctypes.c_int]
    lib.oracle_bwd_input.argtypes = [i64, i64, i64, p, p, p, i64, p, p, ctypes.c_int]
    lib.oracle_grad_weight.argtypes = [i64, i64, i64, p, p, i64, p, p, p, ctypes.c_int]
    lib.oracle_grad_bias.argtypes = [i64, i64, p, p]
    lib.oracle_topology.argtypes = [i64, i64, i64, p, p, p, i64, ctypes.c_uint64,
                                    p, p, p, p, p, p]
    lib.oracle_init_uniform.argtypes = [i64, i64, i64, ctypes.c_uint64, p, p, p, p]
    lib.oracle_splitmix64.argtypes = [ctypes.c_uint64, i64, p]
    lib.oracle_splitmix64.restype = None
    lib.oracle_getrand.argtypes = [ctypes.c_uint64, i64, i64, p]
    lib.oracle_getrand.restype = None
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def build_coo(O, I, rows, cols, vals=None, column_view=True):
    """Appendix B / Table 7: sort to (row, col) order, row offsets, optional CSC view."""
    lib = _load()
    rows, cols = _i32(rows), _i32(cols)
    nnz = rows.size
    vals = None if vals is None else np.ascontiguousarray(vals, dtype=np.float32)
    out = {
        "rows": np.empty(nnz, np.int32), "cols": np.empty(nnz, np.int32),
        "vals": np.empty(nnz, np.float32), "perm": np.empty(nnz, np.int32),
        "row_offsets": np.empty(O + 1, np.int32),
    }
    if column_view:
        out.update(col_perm=np.empty(nnz, np.int32), col_rows=np.empty(nnz, np.int32),
                   col_cols=np.empty(nnz, np.int32), col_offsets=np.empty(I + 1, np.int32))
    st = lib.oracle_build(O, I, nnz, _ptr(rows), _ptr(cols), _ptr(vals),
                          _ptr(out["rows"]), _ptr(out["cols"]), _ptr(out["vals"]),
                          _ptr(out["perm"]), _ptr(out["row_offsets"]),
                          _ptr(out.get("col_perm")), _ptr(out.get("col_rows")),
                          _ptr(out.get("col_cols")), _ptr(out.get("col_offsets")))
    if st:
        raise OracleError(st, "build")
    return out


def fwd(O, I, rows, cols, vals, X, bias=None, nthreads=1):
    """Y = X W^T + b in fp64 (Algorithm 1 plus the nn.Linear bias)."""
    lib = _load()
    rows, cols, vals, X, bias = _i32(rows), _i32(cols), _f64(vals), _f64(X), _f64(bias)
    B = X.shape[0]
    assert X.shape == (B, I)
    Y = np.empty((B, O), np.float64)
    st = lib.oracle_fwd(O, I, rows.size, _ptr(rows), _ptr(cols), _ptr(vals), B,
                        _ptr(X), _ptr(bias), _ptr(Y), nthreads)
    if st:
        raise OracleError(st, "fwd")
    return Y


def bwd_input(O, I, rows, cols, vals, dY, nthreads=1):
    """dX = dY W in fp64 (Section 3.4, W^T by swapped indices)."""
    lib = _load()
    rows, cols, vals, dY = _i32(rows), _i32(cols), _f64(vals), _f64(dY)
    B = dY.shape[0]
    assert dY.shape == (B, O)
    dX = np.empty((B, I), np.float64)
    st = lib.oracle_bwd_input(O, I, rows.size, _ptr(rows), _ptr(cols), _ptr(vals), B,
                              _ptr(dY), _ptr(dX), nthreads)
    if st:
        raise OracleError(st, "bwd_input")
    return dX


def grad_weight(O, I, rows, cols, X, dY, nthreads=1):
    """dW[k] = sum_b dY[b,rows[k]] X[b,cols[k]] in fp64 (Section 3.4 on supp(W))."""
    lib = _load()
    rows, cols, X, dY = _i32(rows), _i32(cols), _f64(X), _f64(dY)
    B = X.shape[0]
    assert X.shape == (B, I) and dY.shape == (B, O)
    dW = np.empty(rows.size, np.float64)
    st = lib.oracle_grad_weight(O, I, rows.size, _ptr(rows), _ptr(cols), B,
                                _ptr(X), _ptr(dY), _ptr(dW), nthreads)
    if st:
        raise OracleError(st, "grad_weight")
    return dW


def grad_bias(dY):
    lib = _load()
    dY = _f64(dY)
    B, O = dY.shape
    db = np.empty(O, np.float64)
    st = lib.oracle_grad_bias(O, B, _ptr(dY), _ptr(db))
    if st:
        raise OracleError(st, "grad_bias")
    return db


def splitmix64(seed: int, n: int) -> np.ndarray:
    lib = _load()
    out = np.empty(n, np.uint64)
    lib.oracle_splitmix64(ctypes.c_uint64(seed), n, _ptr(out))
    return out


def getrand(seed: int, n: int, count: int) -> np.ndarray:
    """Algorithm 2's getrand(n): floor(u * n / 2^64) of successive SplitMix64 outputs u."""
    lib = _load()
    out = np.empty(count, np.int64)
    lib.oracle_getrand(ctypes.c_uint64(seed), n, count, _ptr(out))
    return out


def init_uniform(O, I, nnz, seed):
    """Algorithm 2: nnz distinct positions drawn by rejection (row, then column, per trial) from
    one SplitMix64 stream; returns the sorted rows, cols, row offsets and the trial count."""
    lib = _load()
    out = {"rows": np.empty(nnz, np.int32), "cols": np.empty(nnz, np.int32),
           "row_offsets": np.empty(O + 1, np.int32)}
    trials = ctypes.c_int64(0)
    st = lib.oracle_init_uniform(O, I, nnz, ctypes.c_uint64(seed), _ptr(out["rows"]), _ptr(out["cols"]),
                                 _ptr(out["row_offsets"]), ctypes.byref(trials))
    if st:
        raise OracleError(st, "init_uniform")
    out["trials"] = int(trials.value)
    return out


def topology(O, I, rows, cols, vals, n_prune, seed):
    """Appendix G prune-and-regrow with Algorithm 2 (SplitMix64 getrand); returns a sorted triple."""
    lib = _load()
    rows, cols = _i32(rows), _i32(cols)
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    nnz = rows.size
    out = {"rows": np.empty(nnz, np.int32), "cols": np.empty(nnz, np.int32),
           "vals": np.empty(nnz, np.float32), "row_offsets": np.empty(O + 1, np.int32),
           "pruned": np.empty(max(n_prune, 0), np.int32)}
    trials = ctypes.c_int64(0)
    st = lib.oracle_topology(O, I, nnz, _ptr(rows), _ptr(cols), _ptr(vals), n_prune,
                             ctypes.c_uint64(seed), _ptr(out["rows"]), _ptr(out["cols"]),
                             _ptr(out["vals"]), _ptr(out["row_offsets"]), _ptr(out["pruned"]),
                             ctypes.byref(trials))
    if st:
        raise OracleError(st, "topology")
    out["trials"] = int(trials.value)
    return out
