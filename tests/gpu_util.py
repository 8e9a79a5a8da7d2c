"""Helpers for the GPU parity tests: device layers, tolerance checks, oracle sampling."""
from __future__ import annotations

import contextlib
import functools
import math
import os
import sys

import numpy as np

import oracle
import synth

NTHREADS = max(1, min(16, os.cpu_count() or 1))


def say(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def band_threshold(nnz_min: int | None):
    """Run with SNACK_COO_BAND_MIN_NNZ set (the entry count from which snack_coo_bwd takes its
    row-banded form), or with the library default when nnz_min is None."""
    old = os.environ.get("SNACK_COO_BAND_MIN_NNZ")
    if nnz_min is None:
        os.environ.pop("SNACK_COO_BAND_MIN_NNZ", None)
    else:
        os.environ["SNACK_COO_BAND_MIN_NNZ"] = str(int(nnz_min))
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("SNACK_COO_BAND_MIN_NNZ", None)
        else:
            os.environ["SNACK_COO_BAND_MIN_NNZ"] = old


# banded for every layer / never banded
BANDINGS = {"banded": 1, "unbanded": 1 << 62}


# ---------------------------------------------------------------- tolerances
# fp32: relative L2 <= 1e-5 and max |err| <= 1e-4 * sqrt(n), n = mean reduction
# length of the checked quantity (forward: nnz/O, input gradient: nnz/I, weight
# gradient: the batch).  bf16 activations (outputs rounded to bf16): relative
# L2 <= 1e-2, and max |err| within 2^-8 of the largest magnitude plus the fp32 bound.
def check_close(got, ref, n_reduce: float, what: str, bf16: bool = False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if got.size == 0:
        return
    err = got - ref
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err))
    mx = float(np.max(np.abs(err)))
    bound = 1e-4 * math.sqrt(max(1.0, n_reduce))
    if bf16:
        assert rel <= 1e-2, f"{what}: rel-L2 {rel:.3e} > 1e-2"
        assert mx <= bound + 2.0 ** -8 * float(np.max(np.abs(ref))), f"{what}: max err {mx:.3e}"
    else:
        assert rel <= 1e-5, f"{what}: rel-L2 {rel:.3e} > 1e-5"
        assert mx <= bound, f"{what}: max abs err {mx:.3e} > {bound:.3e}"


# ---------------------------------------------------------------- layers
@functools.lru_cache(maxsize=16)
def named_layer(name: str):
    spec = synth.LAYERS[name]
    L = synth.make_layer(spec)
    return spec, L


def device_layer(L, device):
    import coo_spmm_row_amd as snk
    built = snk.snack_coo_build(L["out_features"], L["in_features"], L["rows"], L["cols"], L["vals"])
    return built, snk.SnackCOO.from_built(built, device)


def acts(seed, B, F, bf16=False):
    a = synth.make_acts(seed, B, F)
    if bf16:
        bits = synth.to_bf16_bits(a)
        return bits, synth.bf16_bits_to_f32(bits)
    return a, a


def to_device(a, device, bf16=False):
    import torch
    if bf16:
        return torch.from_numpy(a.astype(np.uint16).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_device(t):
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(bits)
    return t.cpu().numpy()


# ---------------------------------------------------------------- oracle on samples
def oracle_fwd_rows(built, X, bias, rows_sel):
    """Oracle forward restricted to the output rows rows_sel (all their entries)."""
    off = built["row_offsets"]
    ks = np.concatenate([np.arange(off[r], off[r + 1]) for r in rows_sel]) if len(rows_sel) else np.zeros(0, int)
    remap = np.full(built["out_features"], -1, np.int64)
    remap[rows_sel] = np.arange(len(rows_sel))
    r = remap[built["rows"][ks]]
    b = None if bias is None else bias[rows_sel]
    return oracle.fwd(len(rows_sel), built["in_features"], r, built["cols"][ks], built["vals"][ks], X, b,
                      nthreads=NTHREADS)


def oracle_dx_cols(built, dY, cols_sel):
    """Oracle input gradient restricted to the input columns cols_sel."""
    mask = np.zeros(built["in_features"], bool)
    mask[cols_sel] = True
    ks = np.flatnonzero(mask[built["cols"]])
    remap = np.full(built["in_features"], -1, np.int64)
    remap[cols_sel] = np.arange(len(cols_sel))
    return oracle.bwd_input(built["out_features"], len(cols_sel), built["rows"][ks], remap[built["cols"][ks]],
                            built["vals"][ks], dY, nthreads=NTHREADS)


def oracle_dw_entries(built, X, dY, ks):
    return oracle.grad_weight(built["out_features"], built["in_features"], built["rows"][ks], built["cols"][ks],
                              X, dY, nthreads=NTHREADS)
