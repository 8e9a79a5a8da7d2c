"""The LDS-tiled gather-reduce (forward over the row order, input gradient over the column view
with values in column order) against the fp64 oracle, for every slot width (needs a GPU).

The tiled walk applies to layers of at least 2^20 entries at batches padded to a multiple of 64
whose (key, column block) segments average at least 8 entries.  The cases cover: several column
blocks with a narrower last one, one block, batches that need zero padding (50, 100) and several
64-column batch tiles (128, 192, 256), empty rows and bias-only outputs, rows and columns longer
than the prefetched chunks (the full lines of 'dense_lines'), bf16 activations, and the walk off
(SNACK_COO_TILE=0) giving the same results within tolerance.
"""
import contextlib
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import NTHREADS, acts, check_close, device_layer, from_device, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import coo_spmm_row_amd as snk  # noqa: E402

DEV = torch.device("cuda:0")


@contextlib.contextmanager
def tile_mode(v):
    """SNACK_COO_TILE: '0' off, '1' / '2' / '4' slots per wave, None the library default."""
    old = os.environ.get("SNACK_COO_TILE")
    if v is None:
        os.environ.pop("SNACK_COO_TILE", None)
    else:
        os.environ["SNACK_COO_TILE"] = v
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("SNACK_COO_TILE", None)
        else:
            os.environ["SNACK_COO_TILE"] = old


@pytest.fixture(scope="module")
def layers():
    return {
        # I = 5000: 8 blocks of 625 columns; ~30 entries per segment
        "u3000x5000": synth.random_small_layer(701, 3000, 5000, 1_200_000, "uniform"),
        # I = 7777: 13 blocks of 599 columns (the last one 589); three in four rows empty
        "e1100x7777": synth.random_small_layer(702, 1100, 7777, 1_100_000, "empty_rows"),
        # two full rows and two full columns: segments of a whole block (> 128 entries)
        "d2000x4000": synth.random_small_layer(703, 2000, 4000, 1_000_000, "dense_lines"),
        # I = 600 < one block: a single column block
        "u4000x600": synth.random_small_layer(704, 4000, 600, 1_050_000, "uniform"),
    }


def _fwd_dx(L, B, seed, bf16, mode):
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    Wc = W.to_column_order()
    x_in, x64 = acts(seed, B, I, bf16)
    dy_in, dy64 = acts(seed + 1, B, O, bf16)
    X, dY = to_device(x_in, DEV, bf16), to_device(dy_in, DEV, bf16)
    b = torch.from_numpy(L["bias"]).to(DEV)
    with tile_mode(mode):
        Y = snk.snack_coo_fwd(W, X, b)
        dX = snk.snack_coo_bwd_input(Wc, dY)
    torch.cuda.synchronize()
    r, c, v = built["rows"], built["cols"], built["vals"]
    Yr = oracle.fwd(O, I, r, c, v, x64, L["bias"], nthreads=NTHREADS)
    dXr = oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS)
    check_close(from_device(Y), Yr, nnz / O, f"fwd mode={mode}", bf16)
    check_close(from_device(dX), dXr, nnz / I, f"col-order dX mode={mode}", bf16)
    return Y, dX


@pytest.mark.parametrize("mode", ["1", "2", "4"])
@pytest.mark.parametrize("name", ["u3000x5000", "e1100x7777", "d2000x4000", "u4000x600"])
def test_tiled_fp32_b64(layers, name, mode):
    say(f"tiled {name} B=64 slots={mode}")
    _fwd_dx(layers[name], 64, 7100, False, mode)


@pytest.mark.parametrize("B", [50, 100, 128, 192, 256])
def test_tiled_batches(layers, B):
    say(f"tiled u3000x5000 B={B}")
    _fwd_dx(layers["u3000x5000"], B, 7200 + B, False, None)


@pytest.mark.parametrize("mode", ["1", "4"])
def test_tiled_bf16(layers, mode):
    say(f"tiled e1100x7777 bf16 B=64 slots={mode}")
    _fwd_dx(layers["e1100x7777"], 64, 7300, True, mode)


def test_tiled_deterministic_and_bias_rows(layers):
    """Bit-identical reruns; rows without entries give the bias exactly; scaling X by 2 scales
    Y - b by 2 exactly (no bias, power-of-two scaling is exact in every summation order)."""
    L = layers["e1100x7777"]
    say("tiled determinism / empty rows / exact scaling")
    built, W = device_layer(L, DEV)
    x_in, _ = acts(7400, 64, L["in_features"])
    X = to_device(x_in, DEV)
    b = torch.from_numpy(L["bias"]).to(DEV)
    Y1 = snk.snack_coo_fwd(W, X, b)
    Y2 = snk.snack_coo_fwd(W, X, b)
    assert torch.equal(Y1, Y2)
    empty = np.flatnonzero(np.diff(built["row_offsets"]) == 0)
    assert empty.size > 0
    assert torch.equal(Y1[:, torch.from_numpy(empty).to(DEV)], b[torch.from_numpy(empty).to(DEV)].expand(64, -1))
    Z1 = snk.snack_coo_fwd(W, X)
    Z2 = snk.snack_coo_fwd(W, X * 2.0)
    assert torch.equal(Z2, Z1 * 2.0)


def test_tiled_matches_untiled(layers):
    """The tiled walk and the rowwave walk agree within the fp32 tolerance."""
    L = layers["d2000x4000"]
    say("tiled vs rowwave d2000x4000 B=64")
    Yt, dXt = _fwd_dx(L, 64, 7500, False, None)
    Yr, dXr = _fwd_dx(L, 64, 7500, False, "0")
    nnz = L["nnz"]
    check_close(Yt.cpu().numpy(), Yr.cpu().numpy(), nnz / L["out_features"], "tiled vs rowwave Y")
    check_close(dXt.cpu().numpy(), dXr.cpu().numpy(), nnz / L["in_features"], "tiled vs rowwave dX")


def test_tiled_in_graph(layers):
    """Captured in a HIP graph and replayed several times with eager work in between."""
    L = layers["u3000x5000"]
    say("tiled in a HIP graph")
    built, W = device_layer(L, DEV)
    x_in, _ = acts(7600, 64, L["in_features"])
    X = to_device(x_in, DEV)
    b = torch.from_numpy(L["bias"]).to(DEV)
    ref = snk.snack_coo_fwd(W, X, b)
    ws = torch.empty(max(snk.snack_coo_workspace_bytes(0, W, 64, snk.SNACK_F32), 256), dtype=torch.uint8,
                     device=DEV)
    Y = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        snk.snack_coo_fwd(W, X, b, out=Y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        snk.snack_coo_fwd(W, X, b, out=Y, workspace=ws)
    for _ in range(3):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref)
        _ = X.sum()
