"""Device topology update (prune-and-regrow on the GPU) against the oracle, bit for bit (needs a GPU)."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import coo_spmm_row_amd as snk  # noqa: E402

DEV = torch.device("cuda:0")


def _device_weight(O, I, rows, cols, vals):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    off = np.searchsorted(rows, np.arange(O + 1)).astype(np.int32)
    return snk.SnackCOO(O, I, t(rows), t(cols), t(np.asarray(vals, np.float32)), t(off))


def _check(O, I, rows, cols, vals, p, seed):
    Wn, trials = snk.snack_coo_topology_update_device(_device_weight(O, I, rows, cols, vals), p, seed)
    ref = oracle.topology(O, I, rows, cols, vals, p, seed)
    cv = oracle.build_coo(O, I, ref["rows"], ref["cols"])
    assert trials == ref["trials"], (trials, ref["trials"])
    assert np.array_equal(Wn.rows.cpu().numpy(), ref["rows"])
    assert np.array_equal(Wn.cols.cpu().numpy(), ref["cols"])
    assert np.array_equal(Wn.vals.cpu().numpy().view(np.uint32), ref["vals"].view(np.uint32))
    assert np.array_equal(Wn.row_offsets.cpu().numpy(), ref["row_offsets"])
    for k in ("col_perm", "col_rows", "col_cols", "col_offsets"):
        assert np.array_equal(getattr(Wn, k).cpu().numpy(), cv[k]), k
    return ref


@pytest.mark.parametrize("seed,O,I,nnz,frac", [
    (1, 60, 45, 900, 0.1), (2, 40, 30, 1000, 0.5), (3, 128, 64, 500, 0.1), (4, 7, 300, 60, 0.25),
    (5, 32, 32, 1024, 0.1),   # fully dense: the only free cells are the pruned ones
    (6, 1, 5000, 2000, 0.3), (7, 5000, 1, 3000, 0.3), (8, 333, 777, 5000, 0.0), (9, 50, 40, 0, 0.0),
    (10, 4096, 4096, 838861, 0.1),
])
def test_device_topology_matches_oracle(seed, O, I, nnz, frac):
    say(f"device topology {O}x{I} nnz={nnz} prune {frac}")
    L = synth.random_small_layer(seed, O, I, nnz, "uniform")
    v = L["vals"].copy()
    if nnz:
        v[::13] = np.float32(0.03)   # ties at the cut, both signs
        v[5::13] = np.float32(-0.03)
    p = int(math.floor(frac * nnz))
    for s in (0, 2**63 + 5):
        _check(O, I, L["rows"], L["cols"], v, p, s)


def test_device_topology_many_draw_batches():
    """Batches of 64 draws: the regrowth spans many batches, each marking its cells live."""
    say("device topology, 64 draws per batch")
    with snk.option(snk.OPT_TOPOLOGY_DRAW_BATCH, 64):
        L = synth.random_small_layer(21, 200, 150, 9000, "uniform")
        _check(200, 150, L["rows"], L["cols"], L["vals"], 2000, 1234)
        L = synth.random_small_layer(22, 32, 32, 1000, "uniform")  # nearly full: most draws rejected
        _check(32, 32, L["rows"], L["cols"], L["vals"], 500, 99)


@pytest.mark.parametrize("name", ["gpt2_qkv", "gpt2_fc", "gpt2_proj"])
def test_device_topology_gpt2_shapes_three_steps(name):
    say(f"device topology, three steps on {name}")
    spec = synth.LAYERS[name]
    L = synth.make_layer(spec)
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    rows, cols, vals = L["rows"], L["cols"], L["vals"]
    seeds = synth.seeds_for(spec.config_id, spec.variant)
    for step in range(3):
        ref = _check(O, I, rows, cols, vals, nnz // 10, seeds["topo"](step))
        rows, cols = ref["rows"], ref["cols"]
        vals = (ref["vals"] + np.float32(0.001) * synth.make_acts(step, 1, nnz)[0]).astype(np.float32)


def test_device_topology_llm_scale():
    """10000 x 10000 at 90 % (10M entries), 10 % pruned: the scale the host update is slow at."""
    say("device topology, 10k x 10k 90%")
    L = synth.make_layer(synth.LAYERS["llm90"])
    _check(L["out_features"], L["in_features"], L["rows"], L["cols"], L["vals"], L["nnz"] // 10, 2024)


def test_device_topology_errors():
    W = _device_weight(4, 4, np.array([0, 1], np.int32), np.array([0, 0], np.int32), [1.0, 2.0])
    with pytest.raises(snk.SnackError):
        snk.snack_coo_topology_update_device(W, 3, 0)  # more pruned than stored
    assert snk._lib.snack_coo_topology_workspace_bytes(1 << 18, 1 << 17, 10, 1) == 0  # beyond 2^34 cells
