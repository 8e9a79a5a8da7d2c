"""SnackLinear host side (CPU): Algorithm 2 support, build, persistence, no CPU compute path."""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
from coo_spmm_row_amd.layer import SnackLinear  # noqa: E402


def test_support_is_algorithm_2_and_column_view_is_the_builders():
    layer = SnackLinear(300, 200, sparsity=0.9, seed=5)
    assert layer.nnz == 6000
    ref = oracle.init_uniform(200, 300, 6000, 5)
    assert np.array_equal(layer.rows.numpy(), ref["rows"]) and np.array_equal(layer.cols.numpy(), ref["cols"])
    assert np.array_equal(layer.row_offsets.numpy(), ref["row_offsets"])
    cv = oracle.build_coo(200, 300, ref["rows"], ref["cols"])
    for k in ("col_perm", "col_rows", "col_cols", "col_offsets"):
        assert np.array_equal(getattr(layer, k).numpy(), cv[k]), k
    # stored values ~ N(0, 1/(density*I)): the sample variance is within a few standard errors
    v = layer.vals.detach().numpy().astype(np.float64)
    target = 1.0 / (0.1 * 300)
    assert abs(v.var() / target - 1.0) < 6.0 * math.sqrt(2.0 / v.size)
    b = layer.bias.detach().numpy()
    assert np.all(np.abs(b) <= 1.0 / math.sqrt(300))


def test_same_seed_same_layer_other_seed_other_support():
    a, b, c = SnackLinear(64, 48, 0.8, seed=1), SnackLinear(64, 48, 0.8, seed=1), SnackLinear(64, 48, 0.8, seed=2)
    assert torch.equal(a.rows, b.rows) and torch.equal(a.cols, b.cols) and torch.equal(a.vals, b.vals)
    assert not (torch.equal(a.rows, c.rows) and torch.equal(a.cols, c.cols))


def test_nnz_argument_and_bounds():
    assert SnackLinear(10, 10, nnz=37).nnz == 37
    assert SnackLinear(10, 10, nnz=0).nnz == 0
    with pytest.raises(ValueError):
        SnackLinear(10, 10, nnz=101)
    with pytest.raises(ValueError):
        SnackLinear(10, 10, sparsity=1.0)


def test_save_load_roundtrip(tmp_path):
    layer = SnackLinear(40, 30, 0.7, seed=9)
    p = tmp_path / "w.npz"
    layer.save_npz(p)
    back = SnackLinear.load_npz(p)
    for k in ("rows", "cols", "row_offsets", "col_perm", "col_rows", "col_cols", "col_offsets"):
        assert torch.equal(getattr(layer, k), getattr(back, k)), k
    assert torch.equal(layer.vals, back.vals) and torch.equal(layer.bias, back.bias)
    nb = SnackLinear(40, 30, 0.7, seed=9, bias=False)
    nb.save_npz(tmp_path / "nb.npz")
    assert SnackLinear.load_npz(tmp_path / "nb.npz").bias is None


def test_prune_and_regrow_on_host_matches_the_oracle():
    layer = SnackLinear(50, 40, 0.8, seed=3)
    r, c, v = layer.rows.numpy().copy(), layer.cols.numpy().copy(), layer.vals.detach().numpy().copy()
    trials = layer.prune_and_regrow(0.1, seed=77)
    ref = oracle.topology(40, 50, r, c, v, int(0.1 * r.size), 77)
    assert trials == ref["trials"]
    assert np.array_equal(layer.rows.numpy(), ref["rows"]) and np.array_equal(layer.cols.numpy(), ref["cols"])
    assert np.array_equal(layer.vals.detach().numpy().view(np.uint32), ref["vals"].view(np.uint32))


def test_no_cpu_compute_path():
    layer = SnackLinear(20, 10, 0.5)
    with pytest.raises(ValueError, match="device tensor"):
        layer(torch.randn(3, 20))


def test_column_order_layer_host_side(tmp_path):
    """value_order="col": the same support and values, kept in column-view order with row_to_col the
    inverse of col_perm; host prune-and-regrow and save/load work on row order."""
    row = SnackLinear(60, 45, 0.8, seed=21)
    col = SnackLinear(60, 45, 0.8, seed=21, value_order="col")
    cp = row.col_perm.numpy()
    assert np.array_equal(col.vals.detach().numpy(), row.vals.detach().numpy()[cp])
    assert np.array_equal(col.row_to_col.numpy()[cp], np.arange(cp.size))
    assert torch.equal(col.row_order_vals(), row.vals.detach())
    assert "value_order=col" in repr(col)
    col.save_npz(tmp_path / "c.npz")
    back = SnackLinear.load_npz(tmp_path / "c.npz")  # row order on disk
    assert torch.equal(back.vals, row.vals)
    back_c = SnackLinear.load_npz(tmp_path / "c.npz", value_order="col")
    assert torch.equal(back_c.vals, col.vals) and torch.equal(back_c.row_to_col, col.row_to_col)
    t_row, t_col = row.prune_and_regrow(0.2, seed=7), col.prune_and_regrow(0.2, seed=7)
    assert t_row == t_col
    assert torch.equal(col.rows, row.rows) and torch.equal(col.cols, row.cols)
    assert torch.equal(col.row_order_vals(), row.vals.detach())
    assert np.array_equal(col.vals.detach().numpy(), row.vals.detach().numpy()[row.col_perm.numpy()])
    with pytest.raises(ValueError):
        SnackLinear(10, 10, value_order="diagonal")


def test_deepcopy_and_pickle_after_a_descriptor_view():
    """The layer's cached descriptor view holds raw addresses: deepcopy and pickling leave it out, and
    the copies equal the original."""
    import copy
    import pickle
    for order in ("row", "col"):
        m = SnackLinear(60, 40, sparsity=0.8, seed=5, value_order=order)
        W = m.weight_view()
        assert m.weight_view() is W                      # kept while structure and values stay
        c = copy.deepcopy(m)
        p = pickle.loads(pickle.dumps(m))
        for other in (c, p):
            assert "_view" not in other.__dict__
            assert torch.equal(other.vals, m.vals) and torch.equal(other.rows, m.rows)
            assert other.weight_view().nnz == m.nnz
        m.vals.data = m.vals.data.clone()                # new storage: a new view
        assert m.weight_view() is not W
