"""Seeded synthetic SNACK layers and activations.

Recipe (every draw comes from numpy ``Generator(PCG64(seed))``):

* positions: ``uniform`` draws linear positions q in [0, O*I) and keeps the first
  ``nnz`` distinct ones in draw order (rejection against a bitmap, the way the
  uniform initializer of the SNACK paper, Section 3.3 / Algorithm 2, never
  materialises a dense mask); ``zipf`` gives row r of a seeded rank order a quota
  proportional to rank**-alpha, capped at I with the excess spread over the
  uncapped rows, rounded by largest remainder to exactly ``nnz``; the columns of
  each row are then drawn uniformly without replacement.
* arrays are returned sorted by (row, col), int32 indices, fp32 values.
* vals ~ N(0, variance 1/(density*I)) for the square layers (unit-variance
  outputs), N(0, std 0.02) for the GPT-2-shaped layers; bias ~ N(0, std 0.01);
  X and dY ~ N(0, 1).  bf16 activations are the round-to-nearest-even images of
  the same fp32 draws.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


def nnz_for_density(out_features: int, in_features: int, density_num: int, density_den: int) -> int:
    """round(density * O * I) in integer arithmetic (half rounds up)."""
    total = out_features * in_features * density_num
    return (total + density_den // 2) // density_den


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    out_features: int
    in_features: int
    density_num: int          # density = density_num / density_den
    density_den: int
    batches: tuple
    structure: str = "uniform"   # or "zipf"
    val_std: Optional[float] = None  # None: sqrt(1/(density*I))
    config_id: int = 0
    variant: int = 0

    @property
    def nnz(self) -> int:
        return nnz_for_density(self.out_features, self.in_features, self.density_num, self.density_den)

    @property
    def density(self) -> float:
        return self.density_num / self.density_den


# The workloads: square layers of Section 4 / Appendix D and GPT-2-small shapes of Section 5.
LAYERS = {
    "tiny":        Layer("tiny", 512, 512, 1, 10, (4,), config_id=1),
    "mid":         Layer("mid", 4096, 4096, 1, 20, (1, 8, 32), config_id=2),
    "llm90":       Layer("llm90", 10000, 10000, 1, 10, (1, 16, 64), config_id=3),
    "target95":    Layer("target95", 10000, 10000, 1, 20, (64, 1), config_id=3, variant=1),
    "xs99":        Layer("xs99", 10000, 10000, 1, 100, (1,), config_id=4, variant=0),
    "xs999":       Layer("xs999", 10000, 10000, 1, 1000, (1,), config_id=4, variant=1),
    "xs99_zipf":   Layer("xs99_zipf", 10000, 10000, 1, 100, (1,), structure="zipf", config_id=4, variant=2),
    "xs999_zipf":  Layer("xs999_zipf", 10000, 10000, 1, 1000, (1,), structure="zipf", config_id=4, variant=3),
    "gpt2_qkv":    Layer("gpt2_qkv", 2304, 768, 1, 100, (1024,), val_std=0.02, config_id=5, variant=0),
    "gpt2_fc":     Layer("gpt2_fc", 3072, 768, 1, 100, (1024,), val_std=0.02, config_id=5, variant=1),
    "gpt2_proj":   Layer("gpt2_proj", 768, 3072, 1, 100, (1024,), val_std=0.02, config_id=5, variant=2),
    # the 5000 x 5000 feature-head projection of the GAMLP-shaped workload (Table 6 and its appendix):
    # batch-1 inference at 90 / 95 / 99 % sparsity, training at batch 4096
    "gamlp90":     Layer("gamlp90", 5000, 5000, 1, 10, (1, 4096), config_id=7, variant=0),
    "gamlp95":     Layer("gamlp95", 5000, 5000, 1, 20, (1,), config_id=7, variant=1),
    "gamlp99":     Layer("gamlp99", 5000, 5000, 1, 100, (1,), config_id=7, variant=2),
}


def seeds_for(config_id: int, variant: int = 0):
    """Seed scheme: W = 1000c+v, X_j = 1000c+10+j, dY_j = 1000c+20+j, topology step t = 1000c+100+t."""
    base = 1000 * config_id
    return {
        "W": base + variant,
        "X": lambda j=0: base + 10 + j,
        "dY": lambda j=0: base + 20 + j,
        "topo": lambda t=0: base + 100 + t,
    }


def _uniform_positions(rng: np.random.Generator, total: int, nnz: int) -> np.ndarray:
    """First ``nnz`` distinct draws of a uniform stream over [0, total), in draw order."""
    if nnz > total:
        raise ValueError("nnz exceeds the number of positions")
    seen = np.zeros(total, dtype=bool)
    picked = []
    need = nnz
    while need > 0:
        batch = rng.integers(0, total, size=need + need // 8 + 64, dtype=np.int64)
        _, first = np.unique(batch, return_index=True)
        first.sort()
        batch = batch[first]
        batch = batch[~seen[batch]][:need]
        seen[batch] = True
        picked.append(batch)
        need -= batch.size
    return np.concatenate(picked) if picked else np.zeros(0, dtype=np.int64)


def _zipf_quotas(rows: int, cols: int, nnz: int, alpha: float) -> np.ndarray:
    """Per-rank quotas proportional to rank**-alpha, capped at ``cols``, summing to ``nnz``."""
    weight = np.arange(1, rows + 1, dtype=np.float64) ** (-alpha)
    quota = np.zeros(rows, dtype=np.float64)
    capped = np.zeros(rows, dtype=bool)
    remaining = float(nnz)
    while True:
        free = ~capped
        share = remaining * weight[free] / weight[free].sum()
        over = share > cols
        if not over.any():
            quota[free] = share
            break
        idx = np.flatnonzero(free)[over]
        capped[idx] = True
        quota[idx] = cols
        remaining = nnz - quota[capped].sum()
    base = np.floor(quota).astype(np.int64)
    short = nnz - int(base.sum())
    frac = quota - base
    frac[base >= cols] = -1.0
    order = np.argsort(-frac, kind="stable")
    base[order[:short]] += 1
    assert int(base.sum()) == nnz and base.max() <= cols
    return base


def make_layer(layer: Layer, seed: Optional[int] = None, with_bias: bool = True):
    """Return dict(rows, cols, vals, bias) with entries sorted by (row, col)."""
    O, I, nnz = layer.out_features, layer.in_features, layer.nnz
    if seed is None:
        seed = seeds_for(layer.config_id, layer.variant)["W"]
    rng = np.random.Generator(np.random.PCG64(seed))
    if layer.structure == "uniform":
        pos = np.sort(_uniform_positions(rng, O * I, nnz))
        rows = (pos // I).astype(np.int32)
        cols = (pos % I).astype(np.int32)
    elif layer.structure == "zipf":
        quota = _zipf_quotas(O, I, nnz, 1.5)
        rank_to_row = rng.permutation(O)
        per_row = np.zeros(O, dtype=np.int64)
        per_row[rank_to_row] = quota
        rows = np.repeat(np.arange(O, dtype=np.int32), per_row)
        cols = np.empty(nnz, dtype=np.int32)
        at = 0
        for r in range(O):
            q = int(per_row[r])
            if q:
                cols[at:at + q] = np.sort(rng.choice(I, size=q, replace=False))
                at += q
    else:
        raise ValueError(layer.structure)
    std = layer.val_std if layer.val_std is not None else float(np.sqrt(1.0 / (layer.density * I)))
    vals = (rng.standard_normal(nnz) * std).astype(np.float32)
    bias = (rng.standard_normal(O) * 0.01).astype(np.float32) if with_bias else None
    return {"rows": rows, "cols": cols, "vals": vals, "bias": bias,
            "out_features": O, "in_features": I, "nnz": nnz}


def make_acts(seed: int, batch: int, features: int) -> np.ndarray:
    """fp32 N(0,1) activations, batch-major [batch][features]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((batch, features)).astype(np.float32)


def random_small_layer(seed: int, out_features: int, in_features: int, nnz: int, shape: str = "uniform"):
    """Small hand-shaped layers for edge cases: 'uniform', 'one_row', 'one_col', 'diag', 'empty_rows',
    'dense_lines' (uniform, plus two full rows and two full columns; three other rows and three
    other columns keep only their entries on those full lines), 'skewed_rows' (row = floor(O*u^3)
    for uniform u, so the low rows are dense and the high rows sparse; columns uniform)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    O, I = out_features, in_features
    if shape == "uniform":
        pos = np.sort(_uniform_positions(rng, O * I, nnz))
    elif shape == "one_row":
        r = int(rng.integers(0, O))
        pos = r * I + np.sort(rng.choice(I, size=min(nnz, I), replace=False))
    elif shape == "one_col":
        c = int(rng.integers(0, I))
        pos = np.sort(rng.choice(O, size=min(nnz, O), replace=False)) * I + c
    elif shape == "diag":
        n = min(O, I)
        pos = np.arange(n, dtype=np.int64) * I + np.arange(n, dtype=np.int64)
    elif shape == "empty_rows":
        live = np.sort(rng.choice(O, size=max(1, O // 4), replace=False))
        cand = (live[:, None] * I + np.arange(I)[None, :]).ravel()
        pos = np.sort(rng.choice(cand, size=min(nnz, cand.size), replace=False))
    elif shape == "dense_lines":
        lines_r = rng.choice(O, size=5, replace=False)
        lines_c = rng.choice(I, size=5, replace=False)
        full = np.concatenate([r * I + np.arange(I, dtype=np.int64) for r in lines_r[:2]] +
                              [np.arange(O, dtype=np.int64) * I + c for c in lines_c[:2]])
        pos = np.union1d(_uniform_positions(rng, O * I, nnz), full)
        r_of, c_of = pos // I, pos % I
        drop = np.isin(r_of, lines_r[2:]) | np.isin(c_of, lines_c[2:])
        keep_full = np.isin(r_of, lines_r[:2]) | np.isin(c_of, lines_c[:2])
        pos = pos[~drop | keep_full]
    elif shape == "skewed_rows":
        m = 2 * nnz + 64
        r = np.minimum((O * rng.random(m) ** 3).astype(np.int64), O - 1)
        c = rng.integers(0, I, size=m, dtype=np.int64)
        cand = np.unique(r * I + c)
        pos = np.sort(rng.choice(cand, size=min(nnz, cand.size), replace=False))
    else:
        raise ValueError(shape)
    pos = np.asarray(pos, dtype=np.int64)
    rows = (pos // I).astype(np.int32)
    cols = (pos % I).astype(np.int32)
    vals = rng.standard_normal(pos.size).astype(np.float32)
    bias = (rng.standard_normal(O) * 0.1).astype(np.float32)
    return {"rows": rows, "cols": cols, "vals": vals, "bias": bias,
            "out_features": O, "in_features": I, "nnz": int(pos.size)}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal fp32 values."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
