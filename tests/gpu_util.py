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


def band_threshold(nnz_min: int | None):
    """Run with the entry count from which snack_coo_bwd takes its row-banded form set to nnz_min
    (SNACK_OPT_BAND_MIN_NNZ), or the library default when nnz_min is None."""
    import coo_spmm_row_amd as snk
    return snk.option(snk.OPT_BAND_MIN_NNZ, -1 if nnz_min is None else int(nnz_min))


# banded for every layer / never banded
BANDINGS = {"banded": 1, "unbanded": 1 << 62}


# ---------------------------------------------------------------- tolerances
# fp32: relative L2 <= 1e-5 and |err| <= 1e-4 * sqrt(n) for every element, n the length of
# that element's reduction: a scalar (the mean, for layers whose rows or columns are about
# equally long, or the batch for the weight gradient) or an array broadcast over the output
# (each output feature's own entry count: row_counts / col_counts).  bf16 activations (outputs
# rounded to bf16): relative L2 <= 1e-2, and |err| within 2^-8 of the largest magnitude plus
# the fp32 bound.
def check_close(got, ref, n_reduce, what: str, bf16: bool = False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if got.size == 0:
        return
    err = np.abs(got - ref)
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err))
    bound = 1e-4 * np.sqrt(np.maximum(1.0, np.asarray(n_reduce, dtype=np.float64)))
    if bf16:
        assert rel <= 1e-2, f"{what}: rel-L2 {rel:.3e} > 1e-2"
        bound = bound + 2.0 ** -8 * float(np.max(np.abs(ref)))
    else:
        assert rel <= 1e-5, f"{what}: rel-L2 {rel:.3e} > 1e-5"
    over = err > bound
    if np.any(over):
        at = tuple(np.argwhere(over)[0])
        raise AssertionError(f"{what}: {int(over.sum())} elements over the bound, first {at}: "
                             f"|err| {err[at]:.3e} > {np.broadcast_to(bound, err.shape)[at]:.3e}")


def row_counts(built):
    """Entries per row of W (the forward's reduction length per output feature), shape (1, O)."""
    return np.diff(np.asarray(built["row_offsets"], dtype=np.int64))[None, :]


def col_counts(built):
    """Entries per column of W (the input gradient's reduction length per feature), shape (1, I)."""
    return np.diff(np.asarray(built["col_offsets"], dtype=np.int64))[None, :]


# ---------------------------------------------------------------- layers
@functools.lru_cache(maxsize=16)
def named_layer(name: str):
    spec = synth.LAYERS[name]
    L = synth.make_layer(spec)
    return spec, L


BUILD_KEYS = ("rows", "cols", "perm", "row_offsets", "col_perm", "col_rows", "col_cols", "col_offsets")


def device_layer(L, device):
    """The layer on the device through the library's builder, and the oracle's own build of the
    same input (comparison sort, Appendix B / Table 7) for every reference computation.  The two
    builds must agree bit for bit, so no reference value depends on the library's builder."""
    import coo_spmm_row_amd as snk
    O, I = L["out_features"], L["in_features"]
    built = snk.snack_coo_build(O, I, L["rows"], L["cols"], L["vals"])
    ref = oracle.build_coo(O, I, L["rows"], L["cols"], L["vals"])
    for k in BUILD_KEYS:
        assert np.array_equal(built[k], ref[k]), f"library builder differs from the oracle's: {k}"
    assert np.array_equal(built["vals"].view(np.uint32), ref["vals"].view(np.uint32)), "builder vals"
    ref["out_features"], ref["in_features"], ref["nnz"] = O, I, int(ref["rows"].size)
    return ref, snk.SnackCOO.from_built(built, device)


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
