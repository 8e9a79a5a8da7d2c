"""Library builder (two counting sorts) against the oracle builder (comparison sort), bit-exact (CPU)."""
import numpy as np
import pytest

import coo_spmm_row_amd as snk
import oracle
import synth

KEYS = ["rows", "cols", "perm", "row_offsets", "col_perm", "col_rows", "col_cols", "col_offsets"]


def _compare(O, I, r, c, v):
    a = snk.snack_coo_build(O, I, r, c, v)
    b = oracle.build_coo(O, I, r, c, v)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["vals"].view(np.uint32), b["vals"].view(np.uint32))


@pytest.mark.parametrize("seed,shape,O,I,nnz", [
    (1, "uniform", 50, 40, 300), (2, "one_row", 30, 64, 64), (3, "one_col", 64, 30, 64),
    (4, "diag", 17, 17, 17), (5, "empty_rows", 80, 60, 700), (6, "uniform", 1, 100, 37),
    (7, "uniform", 100, 1, 37), (8, "uniform", 9, 9, 81),
])
def test_builder_matches_oracle_shuffled(seed, shape, O, I, nnz):
    L = synth.random_small_layer(seed, O, I, nnz, shape)
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.permutation(L["nnz"])
    v = L["vals"][p].copy()
    v[::7] = 0.0          # stored zeros are kept
    v[1::11] = -0.0
    _compare(O, I, L["rows"][p], L["cols"][p], v)


def test_builder_tiny_workload_and_zipf_structure():
    L = synth.make_layer(synth.LAYERS["tiny"])
    rng = np.random.Generator(np.random.PCG64(0))
    p = rng.permutation(L["nnz"])
    _compare(512, 512, L["rows"][p], L["cols"][p], L["vals"][p])
    # a power-law row-degree layer at a reduced size
    spec = synth.Layer("zipf_small", 600, 500, 1, 100, (1,), structure="zipf", config_id=9)
    Z = synth.make_layer(spec)
    p = rng.permutation(Z["nnz"])
    _compare(600, 500, Z["rows"][p], Z["cols"][p], Z["vals"][p])


def test_builder_empty_and_sorted_input_is_identity():
    out = snk.snack_coo_build(5, 7, [], [], [])
    assert out["row_offsets"].tolist() == [0] * 6 and out["col_offsets"].tolist() == [0] * 8
    L = synth.random_small_layer(11, 40, 30, 200, "uniform")
    out = snk.snack_coo_build(40, 30, L["rows"], L["cols"], L["vals"])
    assert np.array_equal(out["perm"], np.arange(200))


@pytest.mark.parametrize("args,status", [
    ((4, 4, [0, 1, 0], [1, 2, 1], [1, 2, 3]), "DUPLICATE"),
    ((4, 4, [0, 4], [0, 0], [1, 2]), "INDEX"),
    ((4, 4, [0, -1], [0, 0], [1, 2]), "INDEX"),
    ((4, 4, [0, 1], [0, 9], [1, 2]), "INDEX"),
    ((2, 2, [0, 0, 1, 1, 0], [0, 1, 0, 1, 0], [1] * 5), "SHAPE"),
    ((-1, 4, [], [], []), "SHAPE"),
    ((2**31, 4, [], [], []), "SHAPE"),
])
def test_builder_errors(args, status):
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_build(*args)
    assert e.value.status == status
    # the oracle rejects the same inputs
    with pytest.raises(oracle.OracleError):
        oracle.build_coo(*args)


@pytest.mark.parametrize("name", ["target95", "llm90"])
def test_builder_matches_oracle_full_size_shuffled(name):
    """The 10000 x 10000 layers at 95 % (5M entries) and 90 % (10M entries), fed in a shuffled
    order: the library's counting sorts and the oracle's comparison sort agree bit for bit."""
    L = synth.make_layer(synth.LAYERS[name])
    rng = np.random.Generator(np.random.PCG64(17))
    p = rng.permutation(L["nnz"])
    _compare(L["out_features"], L["in_features"], L["rows"][p], L["cols"][p], L["vals"][p])
