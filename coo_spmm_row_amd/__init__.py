"""SNACK truly-sparse linear layer on MI355X -- Python binding of libsnack_coo.

Thin ctypes marshalling over the C ABI declared in ``include/snack_coo.h``:
every step of the layer runs in the library (HIP kernels for gfx950, host C++
for the builder and the topology update).  PyTorch supplies device memory and
the current HIP stream only.  Importing this package fails if the library has
not been built (``python -m coo_spmm_row_amd.build``).

Source: "Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks on
GPU" (arXiv:2610.04093): Algorithm 1 and Section 3.2 (forward SpMM), Section
3.4 and Appendix F (input and weight gradients), Appendix B Table 7 (COO / CSR
/ CSC), Algorithm 2 and Appendix G (prune-and-regrow).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsnack_coo.so")

SNACK_F32, SNACK_BF16, SNACK_BF16_HW = 0, 1, 2
OP_FWD, OP_BWD_INPUT, OP_GRAD_WEIGHT, OP_BWD = 0, 1, 2, 3
STATUS = {0: "OK", 1: "NULL", 2: "SHAPE", 3: "INDEX", 4: "DUPLICATE", 5: "ALIGN", 6: "DTYPE",
          7: "WORKSPACE", 8: "HIP", 9: "INTERNAL", 10: "NOMEM", 11: "UNSORTED"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m coo_spmm_row_amd.build` "
                      "(hipcc --offload-arch=gfx950); there is no fallback path")

# torch ships its own HIP runtime with the same soname as /opt/rocm's.  Loading
# torch first makes the library bind to that one runtime, so torch's streams
# and events are valid handles for the library's launches.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln}
    except OSError:
        return set()
    return {os.path.realpath(p) for p in paths}


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError("two HIP runtimes are mapped in this process "
                      f"({sorted(_hip_runtimes_mapped())}); import torch before loading libsnack_coo")


class SnackError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.snack_last_error().decode(errors="replace")
        super().__init__(f"{where}: SNACK_ERR_{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class _Desc(ctypes.Structure):
    _fields_ = [("out_features", ctypes.c_int64), ("in_features", ctypes.c_int64),
                ("nnz", ctypes.c_int64), ("rows", ctypes.c_void_p), ("cols", ctypes.c_void_p),
                ("vals", ctypes.c_void_p), ("row_offsets", ctypes.c_void_p),
                ("col_perm", ctypes.c_void_p), ("col_rows", ctypes.c_void_p),
                ("col_cols", ctypes.c_void_p), ("col_offsets", ctypes.c_void_p),
                ("row_to_col", ctypes.c_void_p), ("row_blocks", ctypes.c_void_p),
                ("col_blocks", ctypes.c_void_p)]


_i64, _p, _u64 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64
_D = ctypes.POINTER(_Desc)
_lib.snack_last_error.restype = ctypes.c_char_p
_lib.snack_coo_abi_version.restype = ctypes.c_int
_lib.snack_coo_build.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]
_lib.snack_coo_workspace_bytes.argtypes = [ctypes.c_int, _D, _i64, ctypes.c_int]
_lib.snack_coo_workspace_bytes.restype = ctypes.c_size_t
_lib.snack_coo_fwd.argtypes = [_D, _p, _i64, ctypes.c_int, _p, _p, _p, ctypes.c_size_t, _p]
_lib.snack_coo_fwd_noalloc.argtypes = [_D, _p, _i64, ctypes.c_int, _p, _p, _p]
_lib.snack_coo_bwd_input.argtypes = [_D, _p, _i64, ctypes.c_int, _p, _p, _p, ctypes.c_size_t, _p]
_lib.snack_coo_grad_weight.argtypes = [_D, _p, _p, _i64, ctypes.c_int, _p, _p, ctypes.c_size_t, _p]
_lib.snack_coo_bwd.argtypes = [_D, _p, _p, _i64, ctypes.c_int, _p, _p, _p, _p, ctypes.c_size_t, _p]
_lib.snack_coo_topology_update.argtypes = [_i64, _i64, _i64, _p, _p, _p, _i64, _u64, _p, _p, _p, _p, _p]
_lib.snack_coo_init_uniform.argtypes = [_i64, _i64, _i64, _u64, _p, _p, _p, _p]
_lib.snack_coo_topology_update_device.argtypes = [_D, _i64, _u64, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                  _p, ctypes.c_size_t, _p]
_lib.snack_coo_topology_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
_lib.snack_coo_topology_workspace_bytes.restype = ctypes.c_size_t
_lib.snack_coo_set_probe.argtypes = [_p, _p]
_lib.snack_coo_invert_perm.argtypes = [_p, _i64, _p, _p]
_lib.snack_coo_gather_f32.argtypes = [_p, _p, _i64, _p, _p]
_lib.snack_coo_block_offsets_count.argtypes = [_D, ctypes.c_int]
_lib.snack_coo_block_offsets_count.restype = ctypes.c_int64
_lib.snack_coo_block_offsets.argtypes = [_D, ctypes.c_int, _p, _p]
_lib.snack_coo_bwd_is_fused.argtypes = [_D, _i64, ctypes.c_int]
_lib.snack_coo_set_option.argtypes = [ctypes.c_int, _i64]
_lib.snack_coo_get_option.argtypes = [ctypes.c_int]
_lib.snack_coo_get_option.restype = _i64
SNACK_VIEW_ROWS, SNACK_VIEW_COLS = 0, 1

EXPORTED = ("snack_coo_build", "snack_coo_workspace_bytes", "snack_coo_fwd", "snack_coo_fwd_noalloc",
            "snack_coo_bwd_input", "snack_coo_grad_weight", "snack_coo_bwd", "snack_coo_topology_update", "snack_coo_init_uniform",
            "snack_coo_topology_update_device", "snack_coo_topology_workspace_bytes", "snack_last_error",
            "snack_coo_abi_version", "snack_coo_set_probe", "snack_coo_invert_perm", "snack_coo_gather_f32",
            "snack_coo_block_offsets_count", "snack_coo_block_offsets", "snack_coo_bwd_is_fused",
            "snack_coo_set_option", "snack_coo_get_option")


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(status: int, where: str):
    if status != 0:
        raise SnackError(status, where)


# ------------------------------------------------------------------ host calls
def snack_coo_build(out_features: int, in_features: int, rows, cols, vals=None, column_view: bool = True):
    """Host builder: sort to (row, col), row offsets, optional column view (numpy in, numpy out)."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    nnz = int(rows.size)
    if cols.size != nnz:
        raise ValueError("rows and cols differ in length")
    vals_in = None if vals is None else np.ascontiguousarray(vals, dtype=np.float32)
    out = {"rows": np.empty(nnz, np.int32), "cols": np.empty(nnz, np.int32),
           "vals": np.empty(nnz, np.float32) if vals_in is not None else None,
           "perm": np.empty(nnz, np.int32), "row_offsets": np.empty(out_features + 1, np.int32)}
    if column_view:
        out.update(col_perm=np.empty(nnz, np.int32), col_rows=np.empty(nnz, np.int32),
                   col_cols=np.empty(nnz, np.int32), col_offsets=np.empty(in_features + 1, np.int32))
    st = _lib.snack_coo_build(out_features, in_features, nnz, _np_ptr(rows), _np_ptr(cols), _np_ptr(vals_in),
                              _np_ptr(out["rows"]), _np_ptr(out["cols"]), _np_ptr(out["vals"]),
                              _np_ptr(out["perm"]), _np_ptr(out["row_offsets"]),
                              _np_ptr(out.get("col_perm")), _np_ptr(out.get("col_rows")),
                              _np_ptr(out.get("col_cols")), _np_ptr(out.get("col_offsets")))
    _check(st, "snack_coo_build")
    out["out_features"], out["in_features"], out["nnz"] = out_features, in_features, nnz
    return out


def snack_coo_topology_update(out_features: int, in_features: int, rows, cols, vals, n_prune: int, seed: int):
    """Host prune-and-regrow (Appendix G with Algorithm 2); returns the new sorted triple."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    nnz = int(rows.size)
    out = {"rows": np.empty(nnz, np.int32), "cols": np.empty(nnz, np.int32),
           "vals": np.empty(nnz, np.float32), "row_offsets": np.empty(out_features + 1, np.int32)}
    trials = ctypes.c_int64(0)
    st = _lib.snack_coo_topology_update(out_features, in_features, nnz, _np_ptr(rows), _np_ptr(cols),
                                        _np_ptr(vals), int(n_prune), ctypes.c_uint64(seed),
                                        _np_ptr(out["rows"]), _np_ptr(out["cols"]), _np_ptr(out["vals"]),
                                        _np_ptr(out["row_offsets"]), ctypes.byref(trials))
    _check(st, "snack_coo_topology_update")
    out["trials"] = int(trials.value)
    return out


def snack_coo_init_uniform(out_features: int, in_features: int, nnz: int, seed: int):
    """Host uniform initializer (Algorithm 2): nnz distinct positions, sorted by (row, col), with
    row offsets and the number of trials (numpy out)."""
    out = {"rows": np.empty(nnz, np.int32), "cols": np.empty(nnz, np.int32),
           "row_offsets": np.empty(out_features + 1, np.int32)}
    trials = ctypes.c_int64(0)
    st = _lib.snack_coo_init_uniform(out_features, in_features, nnz, ctypes.c_uint64(seed), _np_ptr(out["rows"]),
                                     _np_ptr(out["cols"]), _np_ptr(out["row_offsets"]), ctypes.byref(trials))
    _check(st, "snack_coo_init_uniform")
    out["trials"] = int(trials.value)
    return out


# ------------------------------------------------------------------ device side
_OPTIONAL_ARRAYS = ("col_perm", "col_rows", "col_cols", "col_offsets", "row_to_col", "row_blocks", "col_blocks")


class SnackCOO:
    """A layer weight resident on one GPU: the sorted triple, row offsets and
    (optionally) the column view, as torch tensors.  ``vals`` may be updated in
    place (same length); the structure arrays must stay as built.

    With ``row_to_col`` (the inverse of ``col_perm``) the values are kept in column-view order:
    ``vals[j]`` belongs to triple entry ``col_perm[j]``, and every dW the library returns for this
    weight is in the same order (see ``to_column_order``).

    ``row_blocks`` / ``col_blocks`` are the segment tables of the tiled kernels (they depend on the
    structure only).  ``blocks="build"`` (the default) builds them on the device when the weight
    is on a GPU; pass tables built for the same structure (or ``blocks=None`` for none: each call
    then builds its table in the workspace)."""

    def __init__(self, out_features, in_features, rows, cols, vals, row_offsets,
                 col_perm=None, col_rows=None, col_cols=None, col_offsets=None, row_to_col=None,
                 row_blocks=None, col_blocks=None, blocks="build"):
        self.out_features, self.in_features = int(out_features), int(in_features)
        self.rows, self.cols, self.vals, self.row_offsets = rows, cols, vals, row_offsets
        self.col_perm, self.col_rows, self.col_cols, self.col_offsets = col_perm, col_rows, col_cols, col_offsets
        self.row_to_col = row_to_col
        self.row_blocks, self.col_blocks = row_blocks, col_blocks
        self.nnz = int(rows.numel())
        self._desc = _Desc()
        self._refresh()
        if blocks == "build" and rows.is_cuda:
            if self.row_blocks is None:
                self.row_blocks = snack_coo_block_offsets(self, SNACK_VIEW_ROWS)
            if self.col_blocks is None and self.col_offsets is not None:
                self.col_blocks = snack_coo_block_offsets(self, SNACK_VIEW_COLS)
            self._refresh()

    @classmethod
    def from_built(cls, built: dict, device, vals=None):
        import torch
        def t(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
        v = built["vals"] if vals is None else vals
        return cls(built["out_features"], built["in_features"], t(built["rows"]), t(built["cols"]),
                   t(np.ascontiguousarray(v, dtype=np.float32)), t(built["row_offsets"]),
                   t(built.get("col_perm")), t(built.get("col_rows")), t(built.get("col_cols")),
                   t(built.get("col_offsets")))

    def _refresh(self):
        d = self._desc
        d.out_features, d.in_features, d.nnz = self.out_features, self.in_features, self.nnz
        d.rows, d.cols, d.vals = self.rows.data_ptr(), self.cols.data_ptr(), self.vals.data_ptr()
        d.row_offsets = self.row_offsets.data_ptr()
        for name in _OPTIONAL_ARRAYS:
            x = getattr(self, name)
            setattr(d, name, None if x is None else x.data_ptr())

    @property
    def desc(self):
        """The C descriptor over the tensors' current addresses (re-read on every access, so
        tensors whose storage was replaced are never passed stale)."""
        self._refresh()
        return ctypes.byref(self._desc)

    @property
    def device(self):
        return self.rows.device

    @property
    def column_order(self) -> bool:
        return self.row_to_col is not None

    def device_bytes(self, blocks: bool = True) -> int:
        """Device bytes of the weight: the triple, row offsets, column view, value permutation and
        (blocks=True) the segment tables."""
        extra = (self.row_blocks, self.col_blocks) if blocks else ()
        return sum(int(x.numel() * x.element_size()) for x in
                   (self.rows, self.cols, self.vals, self.row_offsets, self.col_perm, self.col_rows,
                    self.col_cols, self.col_offsets, self.row_to_col) + extra if x is not None)

    def with_vals(self, vals) -> "SnackCOO":
        """The same structure (and value order) over other values."""
        return SnackCOO(self.out_features, self.in_features, self.rows, self.cols, vals, self.row_offsets,
                        self.col_perm, self.col_rows, self.col_cols, self.col_offsets, self.row_to_col,
                        self.row_blocks, self.col_blocks, blocks=None)

    def to_column_order(self, stream=None) -> "SnackCOO":
        """This weight with its values in column-view order (new ``vals`` and ``row_to_col``
        tensors; the structure arrays are shared).  dW outputs for it come in the same order."""
        import torch
        if self.column_order:
            return self
        if self.col_perm is None:
            raise ValueError("the column view is required")
        rtc = snack_coo_invert_perm(self.col_perm, stream=stream)
        vals = snack_coo_gather_f32(self.vals, self.col_perm, stream=stream)
        W = self.with_vals(vals)
        W.row_to_col = rtc
        return W

    def to_row_order(self, stream=None) -> "SnackCOO":
        """This weight with its values in row (triple) order."""
        if not self.column_order:
            return self
        vals = snack_coo_gather_f32(self.vals, self.row_to_col, stream=stream)
        W = self.with_vals(vals)
        W.row_to_col = None
        return W


# Workspace of the calls made without one: a buffer per (device, stream), grown as needed.  Each
# buffer is recorded on its stream, so when a larger one replaces it the allocator reuses its memory
# only after the work queued there.  Calls under HIP graph capture get a buffer of their own that
# is never released: the graph's replays keep using its address.
_ws_cache = {}
_ws_captured = []


def _dtype_code(t, half_weights: bool = False) -> int:
    """The activation dtype code of tensor t; half_weights selects SNACK_BF16_HW (bf16 weights on
    the matrix cores), which takes bf16 activations."""
    import torch
    if half_weights:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"half_weights takes bfloat16 activations, got {t.dtype}")
        return SNACK_BF16_HW
    if t.dtype == torch.float32:
        return SNACK_F32
    if t.dtype == torch.bfloat16:
        return SNACK_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _stream(device, stream):
    import torch
    return stream if stream is not None else torch.cuda.current_stream(device)


def _stream_handle(device, stream):
    """The hipStream_t of `stream`, else of the current stream of `device` (a torch.device)."""
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(idx))


def _workspace(device, nbytes, workspace=None, stream=None):
    """(pointer, bytes) of the call's workspace: the caller's `workspace` (the library checks its
    size), else the cached buffer of (device, stream) (see _ws_cache) of at least nbytes() bytes."""
    import torch
    if workspace is not None:
        return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    nbytes = nbytes()
    if nbytes == 0:
        return None, 0
    s = _stream(device, stream)
    with torch.cuda.stream(s):
        capturing = torch.cuda.is_current_stream_capturing()
        if capturing:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            _ws_captured.append(buf)
            return ctypes.c_void_p(buf.data_ptr()), buf.numel()
        key = (torch.device(device).index, s.cuda_stream)
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            buf.record_stream(s)
            _ws_cache[key] = buf
    return ctypes.c_void_p(buf.data_ptr()), buf.numel()


def _check_act(t, rows_expected, cols_expected, name):
    if t.dim() != 2 or t.shape[1] != cols_expected or (rows_expected is not None and t.shape[0] != rows_expected):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [batch, {cols_expected}]")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def snack_coo_workspace_bytes(op: int, W: SnackCOO, batch: int, act_dtype: int, desc=None) -> int:
    return int(_lib.snack_coo_workspace_bytes(op, W.desc if desc is None else desc, batch, act_dtype))


def snack_coo_fwd(W: SnackCOO, X, bias=None, out=None, workspace=None, stream=None, half_weights=False):
    """Y = X W^T + bias (Y has X's dtype); half_weights: the weights rounded to bf16 and the
    products on the matrix cores (SNACK_BF16_HW, bf16 X)."""
    import torch
    _check_act(X, None, W.in_features, "X")
    B = X.shape[0]
    dt = _dtype_code(X, half_weights)
    Y = out if out is not None else torch.empty((B, W.out_features), dtype=X.dtype, device=X.device)
    _check_act(Y, B, W.out_features, "Y")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != W.out_features):
        raise ValueError("bias must be float32 [out_features]")
    d = W.desc
    ws, wsn = _workspace(X.device, lambda: snack_coo_workspace_bytes(OP_FWD, W, B, dt, d), workspace, stream)
    st = _lib.snack_coo_fwd(d, ctypes.c_void_p(X.data_ptr()), B, dt,
                            None if bias is None else ctypes.c_void_p(bias.data_ptr()),
                            ctypes.c_void_p(Y.data_ptr()), ws, wsn, _stream_handle(X.device, stream))
    _check(st, "snack_coo_fwd")
    return Y


NOALLOC_SCRATCH_BYTES = 64 << 20


def snack_coo_fwd_noalloc(W: SnackCOO, X, out, bias=None, stream=None, half_weights=False):
    """snack_coo_fwd with its workspace in the library's static device scratch (nothing allocated:
    ``out`` is required).  Calls on one device share the scratch and must not overlap."""
    import torch
    _check_act(X, None, W.in_features, "X")
    B = X.shape[0]
    dt = _dtype_code(X, half_weights)
    _check_act(out, B, W.out_features, "Y")
    if out.dtype != X.dtype:
        raise TypeError("Y must have X's dtype")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != W.out_features):
        raise ValueError("bias must be float32 [out_features]")
    st = _lib.snack_coo_fwd_noalloc(W.desc, ctypes.c_void_p(X.data_ptr()), B, dt,
                                    None if bias is None else ctypes.c_void_p(bias.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()), _stream_handle(X.device, stream))
    _check(st, "snack_coo_fwd_noalloc")
    return out


def snack_coo_bwd_input(W: SnackCOO, dY, out=None, db=None, workspace=None, stream=None, half_weights=False):
    """dX = dY W (dX has dY's dtype); if ``db`` (float32 [O]) is given it receives sum_b dY[b];
    half_weights as for snack_coo_fwd."""
    import torch
    _check_act(dY, None, W.out_features, "dY")
    B = dY.shape[0]
    dt = _dtype_code(dY, half_weights)
    dX = out if out is not None else torch.empty((B, W.in_features), dtype=dY.dtype, device=dY.device)
    _check_act(dX, B, W.in_features, "dX")
    d = W.desc
    ws, wsn = _workspace(dY.device, lambda: snack_coo_workspace_bytes(OP_BWD_INPUT, W, B, dt, d), workspace, stream)
    st = _lib.snack_coo_bwd_input(d, ctypes.c_void_p(dY.data_ptr()), B, dt, ctypes.c_void_p(dX.data_ptr()),
                                  None if db is None else ctypes.c_void_p(db.data_ptr()), ws, wsn,
                                  _stream_handle(dY.device, stream))
    _check(st, "snack_coo_bwd_input")
    return dX


def snack_coo_grad_weight(W: SnackCOO, X, dY, out=None, workspace=None, stream=None, half_weights=False):
    """dW[k] = sum_b dY[b, rows[k]] X[b, cols[k]] (float32 [nnz])."""
    import torch
    _check_act(X, None, W.in_features, "X")
    B = X.shape[0]
    _check_act(dY, B, W.out_features, "dY")
    dt = _dtype_code(X, half_weights)
    if _dtype_code(dY, half_weights) != dt:
        raise TypeError("X and dY must have the same dtype")
    dW = out if out is not None else torch.empty(W.nnz, dtype=torch.float32, device=X.device)
    d = W.desc
    ws, wsn = _workspace(X.device, lambda: snack_coo_workspace_bytes(OP_GRAD_WEIGHT, W, B, dt, d), workspace,
                         stream)
    st = _lib.snack_coo_grad_weight(d, ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(dY.data_ptr()), B, dt,
                                    ctypes.c_void_p(dW.data_ptr()), ws, wsn, _stream_handle(X.device, stream))
    _check(st, "snack_coo_grad_weight")
    return dW


def snack_coo_bwd(W: SnackCOO, X, dY, dx_out=None, dw_out=None, db=None, workspace=None, stream=None,
                  half_weights=False):
    """Both gradients in one call: returns (dX, dW) as snack_coo_bwd_input and
    snack_coo_grad_weight would (dX has dY's dtype, dW float32 [nnz]); ``db`` as for
    snack_coo_bwd_input."""
    import torch
    _check_act(X, None, W.in_features, "X")
    B = X.shape[0]
    _check_act(dY, B, W.out_features, "dY")
    dt = _dtype_code(X, half_weights)
    if _dtype_code(dY, half_weights) != dt:
        raise TypeError("X and dY must have the same dtype")
    dX = dx_out if dx_out is not None else torch.empty((B, W.in_features), dtype=dY.dtype, device=dY.device)
    _check_act(dX, B, W.in_features, "dX")
    dW = dw_out if dw_out is not None else torch.empty(W.nnz, dtype=torch.float32, device=X.device)
    d = W.desc
    ws, wsn = _workspace(X.device, lambda: snack_coo_workspace_bytes(OP_BWD, W, B, dt, d), workspace, stream)
    st = _lib.snack_coo_bwd(d, ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(dY.data_ptr()), B, dt,
                            ctypes.c_void_p(dX.data_ptr()), None if db is None else ctypes.c_void_p(db.data_ptr()),
                            ctypes.c_void_p(dW.data_ptr()), ws, wsn, _stream_handle(X.device, stream))
    _check(st, "snack_coo_bwd")
    return dX, dW


def snack_coo_topology_update_device(W: SnackCOO, n_prune: int, seed: int, workspace=None, stream=None):
    """Prune-and-regrow on the GPU (Appendix G, regrowth by Algorithm 2): returns (the new
    SnackCOO with its column view, the number of draws); equal to the host update + builder."""
    import torch
    dev = W.device
    O, I, n = W.out_features, W.in_features, W.nnz
    i32 = dict(dtype=torch.int32, device=dev)
    rows, cols = torch.empty(n, **i32), torch.empty(n, **i32)
    vals = torch.empty(n, dtype=torch.float32, device=dev)
    row_offsets, col_offsets = torch.empty(O + 1, **i32), torch.empty(I + 1, **i32)
    col_perm, col_rows, col_cols = torch.empty(n, **i32), torch.empty(n, **i32), torch.empty(n, **i32)
    need = int(_lib.snack_coo_topology_workspace_bytes(O, I, n, int(n_prune)))
    if need == 0:  # invalid sizes (the message says which)
        _check(2, "snack_coo_topology_workspace_bytes")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    trials = ctypes.c_int64(0)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = _lib.snack_coo_topology_update_device(W.desc, int(n_prune), ctypes.c_uint64(seed), p(rows), p(cols),
                                               p(vals), p(row_offsets), p(col_perm), p(col_rows), p(col_cols),
                                               p(col_offsets), ctypes.byref(trials), p(ws),
                                               ws.numel() * ws.element_size(), _stream_handle(dev, stream))
    _check(st, "snack_coo_topology_update_device")
    return SnackCOO(O, I, rows, cols, vals, row_offsets, col_perm, col_rows, col_cols, col_offsets), int(trials.value)


def snack_coo_invert_perm(perm, out=None, stream=None):
    """inv[perm[j]] = j on the device (int32); perm must be a permutation of 0..n-1."""
    import torch
    if perm.dtype != torch.int32 or not perm.is_cuda or not perm.is_contiguous():
        raise ValueError("perm must be a contiguous int32 device tensor")
    inv = out if out is not None else torch.empty_like(perm)
    st = _lib.snack_coo_invert_perm(ctypes.c_void_p(perm.data_ptr()), perm.numel(), ctypes.c_void_p(inv.data_ptr()),
                                    _stream_handle(perm.device, stream))
    _check(st, "snack_coo_invert_perm")
    return inv


def snack_coo_gather_f32(src, idx, out=None, stream=None):
    """dst[j] = src[idx[j]] on the device (float32 values, int32 indices)."""
    import torch
    if src.dtype != torch.float32 or idx.dtype != torch.int32 or not src.is_cuda or not idx.is_cuda:
        raise ValueError("src must be float32 and idx int32, both on the device")
    if not src.is_contiguous() or not idx.is_contiguous():
        raise ValueError("src and idx must be contiguous")
    dst = out if out is not None else torch.empty(idx.numel(), dtype=torch.float32, device=src.device)
    st = _lib.snack_coo_gather_f32(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(idx.data_ptr()), idx.numel(),
                                   ctypes.c_void_p(dst.data_ptr()), _stream_handle(src.device, stream))
    _check(st, "snack_coo_gather_f32")
    return dst


def snack_coo_block_offsets(W: SnackCOO, view: int, out=None, stream=None):
    """The segment table of one view (SNACK_VIEW_ROWS or SNACK_VIEW_COLS) on the device (int32)."""
    import torch
    n = int(_lib.snack_coo_block_offsets_count(W.desc, view))
    if n < 0:
        _check(6, "snack_coo_block_offsets_count")
    t = out if out is not None else torch.empty(max(n, 1), dtype=torch.int32, device=W.device)
    if t.numel() < n or t.dtype != torch.int32 or not t.is_cuda:
        raise ValueError(f"out must be an int32 device tensor of at least {n} entries")
    st = _lib.snack_coo_block_offsets(W.desc, view, ctypes.c_void_p(t.data_ptr()), _stream_handle(W.device, stream))
    _check(st, "snack_coo_block_offsets")
    return t


def snack_coo_bwd_is_fused(W: SnackCOO, batch: int, act_dtype: int = 0) -> bool:
    """Whether snack_coo_bwd takes both gradients in one pass (True) or two tiled passes (False)."""
    r = int(_lib.snack_coo_bwd_is_fused(W.desc, int(batch), int(act_dtype)))
    if r < 0:
        _check(-r, "snack_coo_bwd_is_fused")
    return r == 1


def snack_coo_set_probe(start_event=None, stop_event=None):
    """Arm (two torch.cuda.Event with timing, already recorded once) or disarm (no args) the
    main-kernel timing probe for device calls made from this thread."""
    a = None if start_event is None else ctypes.c_void_p(start_event.cuda_event)
    b = None if stop_event is None else ctypes.c_void_p(stop_event.cuda_event)
    _check(_lib.snack_coo_set_probe(a, b), "snack_coo_set_probe")


def abi_version() -> int:
    return int(_lib.snack_coo_abi_version())


# Kernel-selection overrides (snack_coo_set_option): for tests and measurement only.
OPT_TILE, OPT_BWD_FORM, OPT_BAND_MIN_NNZ, OPT_TOPOLOGY_DRAW_BATCH, OPT_BF16_DW_MFMA = 0, 1, 2, 3, 4


def set_option(opt: int, value: int) -> None:
    """Process-wide override of a kernel choice (-1: the library's own)."""
    _check(_lib.snack_coo_set_option(int(opt), int(value)), "snack_coo_set_option")


def get_option(opt: int) -> int:
    return int(_lib.snack_coo_get_option(int(opt)))


@contextlib.contextmanager
def option(opt: int, value: int):
    """set_option for the duration of a with-block, then the previous value again."""
    old = get_option(opt)
    set_option(opt, value)
    try:
        yield
    finally:
        set_option(opt, old)
