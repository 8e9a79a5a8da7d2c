"""Library topology update (host C++) against the oracle, bit-exact (CPU)."""
import math

import numpy as np
import pytest

import coo_spmm_row_amd as snk
import oracle
import synth


def _same(a, b):
    for k in ("rows", "cols", "row_offsets"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["vals"].view(np.uint32), b["vals"].view(np.uint32))
    assert a["trials"] == b["trials"]


@pytest.mark.parametrize("seed,O,I,nnz,frac", [
    (1, 60, 45, 900, 0.1), (2, 40, 30, 1000, 0.5), (3, 128, 64, 500, 0.1), (4, 7, 300, 60, 0.25),
    (5, 32, 32, 1024, 0.1),   # fully dense: the only free cells are the pruned ones
])
def test_topology_matches_oracle(seed, O, I, nnz, frac):
    L = synth.random_small_layer(seed, O, I, nnz, "uniform")
    v = L["vals"].copy()
    v[::13] = np.float32(0.03)   # ties at the cut
    v[5::13] = np.float32(-0.03)
    p = int(math.floor(frac * nnz))
    for s in (0, 1, 2**63 + 5):
        _same(snk.snack_coo_topology_update(O, I, L["rows"], L["cols"], v, p, s),
              oracle.topology(O, I, L["rows"], L["cols"], v, p, s))


@pytest.mark.parametrize("name", ["gpt2_qkv", "gpt2_fc", "gpt2_proj"])
def test_topology_gpt2_shapes_three_steps(name):
    spec = synth.LAYERS[name]
    L = synth.make_layer(spec)
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    rows, cols, vals = L["rows"], L["cols"], L["vals"]
    seeds = synth.seeds_for(spec.config_id, spec.variant)
    for step in range(3):
        p = nnz // 10
        a = snk.snack_coo_topology_update(O, I, rows, cols, vals, p, seeds["topo"](step))
        b = oracle.topology(O, I, rows, cols, vals, p, seeds["topo"](step))
        _same(a, b)
        # next step starts from the updated layer with perturbed values
        rows, cols = a["rows"], a["cols"]
        vals = (a["vals"] + np.float32(0.001) * synth.make_acts(step, 1, nnz)[0]).astype(np.float32)


def test_topology_errors():
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_topology_update(4, 4, [1, 0], [0, 0], [1.0, 2.0], 1, 0)
    assert e.value.status == "UNSORTED"
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_topology_update(4, 4, [0, 0], [1, 1], [1.0, 2.0], 1, 0)
    assert e.value.status == "UNSORTED"
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_topology_update(4, 4, [0, 5], [1, 1], [1.0, 2.0], 1, 0)
    assert e.value.status == "INDEX"
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_topology_update(4, 4, [0, 1], [1, 1], [1.0, 2.0], 3, 0)
    assert e.value.status == "SHAPE"
    out = snk.snack_coo_topology_update(4, 4, [0, 1], [1, 1], [1.0, 2.0], 0, 0)
    assert out["rows"].tolist() == [0, 1] and out["trials"] == 0


# ---------------------------------------------------------------- uniform initializer (Algorithm 2)
@pytest.mark.parametrize("O,I,nnz", [(60, 45, 900), (32, 32, 1024), (1, 500, 77), (500, 1, 500), (512, 512, 26214),
                                     (768, 2304, 17695), (333, 777, 0)])
def test_init_uniform_matches_oracle(O, I, nnz):
    for s in (0, 11, 2**64 - 1):
        a = snk.snack_coo_init_uniform(O, I, nnz, s)
        b = oracle.init_uniform(O, I, nnz, s)
        for k in ("rows", "cols", "row_offsets"):
            assert np.array_equal(a[k], b[k]), k
        assert a["trials"] == b["trials"]


def test_init_uniform_errors():
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_init_uniform(4, 4, 17, 0)  # more positions than cells
    assert e.value.status == "SHAPE"
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_init_uniform(0, 4, 0, 0)
    assert e.value.status == "SHAPE"
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_init_uniform(1 << 18, 1 << 17, 10, 0)  # beyond the 2^34-cell bitmap
    assert e.value.status == "SHAPE"
