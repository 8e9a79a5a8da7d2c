"""PyTorch drop-in for ``nn.Linear`` over the SNACK C ABI.

SNACK ("Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks on GPU"),
Section 3.5 and Appendix F: the layer keeps its weight as the COO triple on the device
for its whole life, wires forward and backward through a custom autograd function (the
SpMM for the output and the input gradient, the sparse outer product for the weight
gradient), and draws its initial support with the uniform initializer of Algorithm 2.
Every product runs in the library's kernels; this module only marshals tensors.

Readings where the pages leave a step open:
  * stored values start as N(0, 1 / (density * in_features)) (the variance-preserving
    scale for a fan-in of density * in_features), the bias as nn.Linear's
    U(-1/sqrt(in_features), 1/sqrt(in_features));
  * prune-and-regrow (Appendix G) keeps the number of stored entries; regrown entries
    start at 0, and optimizer state kept per entry no longer lines up with the new
    support (the caller resets it).

value_order="col" keeps ``vals`` (and so its gradient and any per-entry optimizer state) in
column-view order for the layer's whole life: the backward pass then reads the values and writes
their gradient contiguously, and the forward pass reads the values through ``row_to_col`` instead.
The products are the same; save_npz always writes row (triple) order.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch
from torch import nn

from . import (SnackCOO, snack_coo_build, snack_coo_bwd, snack_coo_bwd_input, snack_coo_fwd,
               snack_coo_gather_f32, snack_coo_grad_weight, snack_coo_init_uniform, snack_coo_topology_update,
               snack_coo_topology_update_device)

_STRUCT = ("rows", "cols", "row_offsets", "col_perm", "col_rows", "col_cols", "col_offsets")
_ORDERS = ("row", "col")


class SnackLinearFunction(torch.autograd.Function):
    """Y = X W^T + b with W a SnackCOO whose ``vals`` is the ``vals`` argument.

    Backward: dX = dY W (SpMM over the column view), dW[k] = sum_b dY[b, rows[k]] X[b, cols[k]]
    on the support only, db = sum_b dY[b]; both products from one fused call when both are needed.
    """

    @staticmethod
    def forward(ctx, X: torch.Tensor, vals: torch.Tensor, bias: Optional[torch.Tensor], weight: SnackCOO,
                half_weights: bool = False):
        hw = bool(half_weights) and X.dtype == torch.bfloat16
        Y = snack_coo_fwd(weight, X, bias, half_weights=hw)
        ctx.save_for_backward(X)
        ctx.weight = weight
        ctx.hw = hw
        return Y

    @staticmethod
    def backward(ctx, dY: torch.Tensor):
        (X,) = ctx.saved_tensors
        W, hw = ctx.weight, ctx.hw
        need_x, need_v, need_b = ctx.needs_input_grad[:3]
        dY = dY.to(X.dtype).contiguous()
        db = torch.empty(W.out_features, dtype=torch.float32, device=dY.device) if need_b else None
        dX = dW = None
        if need_v and (need_x or need_b):
            dX, dW = snack_coo_bwd(W, X, dY, db=db, half_weights=hw)
        elif need_v:
            dW = snack_coo_grad_weight(W, X, dY, half_weights=hw)
        elif need_x or need_b:
            dX = snack_coo_bwd_input(W, dY, db=db, half_weights=hw)
        return (dX if need_x else None), dW, db, None, None


class SnackLinear(nn.Module):
    """Truly sparse linear layer: ``out_features x in_features`` weight held as a sorted COO
    triple with its column view (never dense), ``vals`` the trainable stored values.

    Give either ``sparsity`` (fraction of zero weights) or ``nnz``.  Inputs are ``[..., in_features]``
    in float32 or bfloat16 on the layer's GPU (bfloat16 in, bfloat16 out, fp32 accumulation);
    there is no CPU path.  ``half_weights`` (bfloat16 inputs only): the stored values are rounded
    to bfloat16 as the kernels read them and the forward and input-gradient products run on the
    matrix cores (SNACK_BF16_HW); the trainable values stay fp32.
    """

    def __init__(self, in_features: int, out_features: int, sparsity: float = 0.9, bias: bool = True,
                 seed: int = 0, nnz: Optional[int] = None, device=None, value_order: str = "row",
                 half_weights: bool = False):
        super().__init__()
        if value_order not in _ORDERS:
            raise ValueError(f"value_order must be one of {_ORDERS}")
        self.value_order = value_order
        self.half_weights = bool(half_weights)
        self.in_features, self.out_features = int(in_features), int(out_features)
        cells = self.in_features * self.out_features
        if nnz is None:
            if not 0.0 <= sparsity < 1.0:
                raise ValueError("sparsity must be in [0, 1)")
            nnz = int(round((1.0 - sparsity) * cells))
        if not 0 <= nnz <= cells:
            raise ValueError(f"nnz={nnz} outside [0, {cells}]")
        topo = snack_coo_init_uniform(self.out_features, self.in_features, int(nnz), int(seed))
        density = max(nnz, 1) / cells
        g = np.random.Generator(np.random.PCG64(int(seed) + 1))
        vals = (g.standard_normal(nnz) / math.sqrt(density * self.in_features)).astype(np.float32)
        self._set_topology(topo["rows"], topo["cols"], vals, device)
        if bias:
            bound = 1.0 / math.sqrt(self.in_features)
            b = g.uniform(-bound, bound, self.out_features).astype(np.float32)
            self.bias = nn.Parameter(torch.from_numpy(b).to(device))
        else:
            self.register_parameter("bias", None)

    @classmethod
    def from_triple(cls, out_features: int, in_features: int, rows, cols, vals, bias=None,
                    device=None, value_order: str = "row") -> "SnackLinear":
        """A layer over a given support and values (host arrays in any order; the builder sorts
        them and rejects duplicates), with the given bias or none."""
        if value_order not in _ORDERS:
            raise ValueError(f"value_order must be one of {_ORDERS}")
        layer = cls.__new__(cls)
        nn.Module.__init__(layer)
        layer.value_order = value_order
        layer.in_features, layer.out_features = int(in_features), int(out_features)
        layer._set_topology(rows, cols, vals, device)
        if bias is not None:
            layer.bias = nn.Parameter(torch.from_numpy(np.array(bias, np.float32)).to(device))
        else:
            layer.register_parameter("bias", None)
        return layer

    # ---------------------------------------------------------------- structure
    def _set_topology(self, rows, cols, vals, device=None):
        """Build the sorted triple and column view on the host and move them to `device`; with
        value_order "col" the values are permuted into column order here (host, set-up only)."""
        built = snack_coo_build(self.out_features, self.in_features, rows, cols, vals, column_view=True)
        if device is None:
            device = self.vals.device if hasattr(self, "vals") else torch.device("cpu")
        v = built["vals"]
        if self.value_order == "col":
            cp = built["col_perm"]
            rtc = np.empty_like(cp)
            rtc[cp] = np.arange(cp.size, dtype=np.int32)
            built["row_to_col"] = rtc
            v = v[cp]
        for name in _STRUCT + (("row_to_col",) if self.value_order == "col" else ()):
            self._set_buffer(name, torch.from_numpy(np.ascontiguousarray(built[name])).to(device))
        self._set_vals(torch.from_numpy(np.ascontiguousarray(v)).to(device))

    def _set_buffer(self, name, t):
        if name in _STRUCT:  # a new structure: the segment tables are rebuilt on next use
            self._struct_version = getattr(self, "_struct_version", 0) + 1
        if name in self._buffers:
            self._buffers[name] = t
        else:
            self.register_buffer(name, t)

    def _set_vals(self, v):
        if "vals" in self._parameters:
            self.vals.data = v
        else:
            self.vals = nn.Parameter(v)

    @property
    def nnz(self) -> int:
        return int(self.rows.numel())

    def _blocks_key_now(self):
        return (getattr(self, "_struct_version", 0), self.rows.data_ptr(), self.col_rows.data_ptr(), self.nnz,
                str(self.rows.device))

    def weight_view(self) -> SnackCOO:
        """The library descriptor over the current tensors.  It is kept while the structure and the
        storage of ``vals`` stay the same (in-place updates of the values keep it valid); the
        segment tables of the tiled kernels are built once per structure and device."""
        key = self._blocks_key_now()
        if getattr(self, "_blocks_key", None) != key:
            self._blocks = (None, None)
            self._blocks_key = key
            self._view = None
            if self.rows.is_cuda:
                W = SnackCOO(self.out_features, self.in_features, self.rows, self.cols, self.vals.detach(),
                             self.row_offsets, self.col_perm, self.col_rows, self.col_cols, self.col_offsets)
                self._blocks = (W.row_blocks, W.col_blocks)
        view = getattr(self, "_view", None)
        if view is None or view[0] != self.vals.data_ptr():
            W = SnackCOO(self.out_features, self.in_features, self.rows, self.cols, self.vals.detach(),
                         self.row_offsets, self.col_perm, self.col_rows, self.col_cols, self.col_offsets,
                         self._buffers.get("row_to_col") if self.value_order == "col" else None,
                         self._blocks[0], self._blocks[1], blocks=None)
            self._view = view = (self.vals.data_ptr(), W)
        return view[1]

    def row_order_vals(self) -> torch.Tensor:
        """The values in row (triple) order, whatever the layer keeps."""
        v = self.vals.detach()
        if self.value_order != "col":
            return v
        if v.is_cuda:
            return snack_coo_gather_f32(v, self.row_to_col)
        return torch.from_numpy(v.numpy()[self.row_to_col.numpy()])

    def __getstate__(self):
        """Pickling and deepcopy leave out the cached descriptor view (it holds raw device
        addresses); the copy builds its own on first use."""
        state = self.__dict__.copy()
        state.pop("_view", None)
        return state

    # ---------------------------------------------------------------- compute
    def forward(self, X: torch.Tensor) -> torch.Tensor:
        if X.shape[-1] != self.in_features:
            raise ValueError(f"input has {X.shape[-1]} features, expected {self.in_features}")
        lead = X.shape[:-1]
        X2 = X.reshape(-1, self.in_features).contiguous()
        Y = SnackLinearFunction.apply(X2, self.vals, self.bias, self.weight_view(), getattr(self, "half_weights", False))
        return Y.reshape(*lead, self.out_features)

    # ---------------------------------------------------------------- topology update (Appendix G)
    @torch.no_grad()
    def prune_and_regrow(self, fraction: float = 0.1, seed: int = 0, on_device: Optional[bool] = None) -> int:
        """Prune the floor(fraction * nnz) smallest |vals| and regrow as many empty positions with
        Algorithm 2; returns the number of trials.  On a GPU layer the update runs on the device
        (snack_coo_topology_update_device) unless on_device=False, which takes the host path; both
        give the same support, values and trial count."""
        n_prune = int(math.floor(fraction * self.nnz))
        if on_device is None:
            on_device = self.vals.is_cuda
        if on_device:
            W, trials = snack_coo_topology_update_device(self.weight_view().to_row_order(), n_prune, int(seed))
            if self.value_order == "col":
                W = W.to_column_order()
                self._set_buffer("row_to_col", W.row_to_col)
            for name in _STRUCT:
                self._set_buffer(name, getattr(W, name))
            self.vals.data = W.vals
            self._blocks = (W.row_blocks, W.col_blocks)  # built for the new structure
            self._blocks_key = self._blocks_key_now()
            self._view = None
            return trials
        out = snack_coo_topology_update(self.out_features, self.in_features, self.rows.cpu().numpy(),
                                        self.cols.cpu().numpy(), self.row_order_vals().cpu().numpy(), n_prune,
                                        int(seed))
        self._set_topology(out["rows"], out["cols"], out["vals"], self.vals.device)
        return out["trials"]

    # ---------------------------------------------------------------- persistence
    def save_npz(self, path) -> None:
        """The COO triple (and bias) as an .npz file (plain arrays, no pickles)."""
        arrays = {"shape": np.array([self.out_features, self.in_features], np.int64),
                  "rows": self.rows.cpu().numpy(), "cols": self.cols.cpu().numpy(),
                  "vals": self.row_order_vals().cpu().numpy()}
        if self.bias is not None:
            arrays["bias"] = self.bias.detach().cpu().numpy()
        np.savez(path, **arrays)

    @classmethod
    def load_npz(cls, path, device=None, value_order: str = "row") -> "SnackLinear":
        with np.load(path, allow_pickle=False) as f:
            O, I = (int(x) for x in f["shape"])
            return cls.from_triple(O, I, f["rows"], f["cols"], f["vals"],
                                   f["bias"] if "bias" in f.files else None, device, value_order)

    def extra_repr(self) -> str:
        cells = self.in_features * self.out_features
        return (f"in_features={self.in_features}, out_features={self.out_features}, nnz={self.nnz} "
                f"(sparsity {1.0 - self.nnz / max(cells, 1):.4f}), bias={self.bias is not None}, "
                f"value_order={self.value_order}")
