"""Seeded synthetic inputs for the SNACK COO layer (shared by tests, smoke and bench).

This module draws random numbers and lays them out; it holds none of the layer's
arithmetic (no products, no sums over non-zeros, no sorting logic of the method).
Both the oracle side and the HIP side receive the arrays it produces.

Workloads follow the shapes of the SNACK paper (arXiv:2610.04093, "Beyond Masked
Sparsity: SNACK Enables Truly Sparse Neural Networks on GPU"): square layers at
90-99.9 % sparsity with small batches (Section 4.1, Table 2; Appendix D.2,
Tables 11-12), and GPT-2-small-shaped MLP/QKV layers (Section 5).  Positions are
drawn uniformly without replacement, as the uniform initializer of Section 3.3
(Algorithm 2) does, or with Zipf-distributed row degrees to stress load balance.
"""
from .layers import (  # noqa: F401
    Layer,
    LAYERS,
    make_layer,
    make_acts,
    nnz_for_density,
    to_bf16_bits,
    bf16_bits_to_f32,
    seeds_for,
    random_small_layer,
)
