"""The LDS-tiled kernels (forward over the row order, input gradient over the column view with
values in either order, weight gradient over the row view) against the fp64 oracle (needs a GPU).

The tiled walks apply to layers of at least 2^19 entries at batches padded to a multiple of 16
(batch tiles of 64 columns where the padded batch allows, else 32 or 16; the weight gradient only
at multiples of 64) whose (key, column block) segments average at least 8 entries.  The cases
cover: several column blocks with a narrower last one, one block, every tile width, batches that
need zero padding (50, 100) and several batch tiles (48, 96, 128, 192, 256, and 512 to 4096 on
the 5000 x 5000 layer), empty rows and
bias-only outputs, rows and columns longer than the prefetched chunks (the full lines of
'dense_lines'), bf16 activations, and the walks off (SNACK_OPT_TILE = 0) giving the same results
within tolerance.
"""
import contextlib
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (NTHREADS, acts, check_close, col_counts, device_layer, from_device, named_layer, row_counts,
                      say, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import coo_spmm_row_amd as snk  # noqa: E402

DEV = torch.device("cuda:0")


def tile_mode(v):
    """The tiled kernels: '0' off (SNACK_OPT_TILE = 0), None the library default (on)."""
    return snk.option(snk.OPT_TILE, -1 if v is None else int(v))


@pytest.fixture(scope="module")
def layers():
    # every layer holds at least 2^20 entries, the tiled kernels' threshold
    return {
        # I = 5000: 8 blocks of 625 columns; ~30 entries per segment
        "u3000x5000": synth.random_small_layer(701, 3000, 5000, 1_200_000, "uniform"),
        # I = 7777: 13 blocks of 599 columns (the last one 589); three in four rows empty
        "e1100x7777": synth.random_small_layer(702, 1100, 7777, 1_100_000, "empty_rows"),
        # two full rows and two full columns: segments of a whole block (> 128 entries)
        "d2000x4000": synth.random_small_layer(703, 2000, 4000, 1_100_000, "dense_lines"),
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


@pytest.mark.parametrize("B", [16, 32, 64])
@pytest.mark.parametrize("name", ["u3000x5000", "e1100x7777", "d2000x4000", "u4000x600"])
def test_tiled_fp32(layers, name, B):
    say(f"tiled {name} B={B}")
    _fwd_dx(layers[name], B, 7100 + B, False, None)


@pytest.mark.parametrize("B", [13, 30, 48, 50, 96, 100, 128, 192, 256])
def test_tiled_batches(layers, B):
    say(f"tiled u3000x5000 B={B}")
    _fwd_dx(layers["u3000x5000"], B, 7200 + B, False, None)


@pytest.mark.parametrize("B", [16, 64])
def test_tiled_bf16(layers, B):
    say(f"tiled e1100x7777 bf16 B={B}")
    _fwd_dx(layers["e1100x7777"], B, 7300 + B, True, None)


def test_tiled_row_order_input_gradient(layers):
    """The input gradient with values in row order (read through col_perm), at every tile width."""
    L = layers["e1100x7777"]
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    for B in (16, 32, 64, 128):
        say(f"tiled row-order dX e1100x7777 B={B}")
        dy_in, dy64 = acts(7350 + B, B, O)
        dX = snk.snack_coo_bwd_input(W, to_device(dy_in, DEV))
        torch.cuda.synchronize()
        ref = oracle.bwd_input(O, I, built["rows"], built["cols"], built["vals"], dy64, nthreads=NTHREADS)
        check_close(dX.cpu().numpy(), ref, nnz / I, f"row-order dX B={B}")


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


def _ref_blocks(offs, gidx, n):
    """Segment lists (numpy): for block j (gather indices [j w, j w + w)) and list position p the
    record {key, start, end, 0}; within each window of 32 positions the window's keys by decreasing
    segment length, equal lengths by increasing key."""
    nb = max(1, -(-n // 638))
    w = max(1, -(-n // nb))
    keys = offs.size - 1
    bounds = np.empty((keys, nb + 1), np.int64)
    for key in range(keys):
        a, e = int(offs[key]), int(offs[key + 1])
        bounds[key] = a + np.searchsorted(gidx[a:e], np.arange(nb + 1) * w, side="left")
        bounds[key, nb] = e
    rec = np.zeros((nb, keys, 4), np.int64)
    for j in range(nb):
        lens = bounds[:, j + 1] - bounds[:, j]
        for w0 in range(0, keys, 32):
            ks = np.arange(w0, min(keys, w0 + 32))
            order = ks[np.lexsort((ks, -lens[ks]))]
            rec[j, w0:w0 + ks.size, 0] = order
            rec[j, w0:w0 + ks.size, 1] = bounds[order, j]
            rec[j, w0:w0 + ks.size, 2] = bounds[order, j + 1]
    return rec.ravel()


@pytest.mark.parametrize("name", ["e1100x7777", "d2000x4000", "u4000x600"])
def test_block_tables_exact(layers, name):
    """snack_coo_block_offsets (both views) equals a per-key search and sort, bit for bit."""
    L = layers[name]
    say(f"segment tables {name}")
    built, W = device_layer(L, DEV)
    O, I = L["out_features"], L["in_features"]
    rb = W.row_blocks.cpu().numpy().astype(np.int64)
    cb = W.col_blocks.cpu().numpy().astype(np.int64)
    assert np.array_equal(rb, _ref_blocks(built["row_offsets"], built["cols"], I))
    assert np.array_equal(cb, _ref_blocks(built["col_offsets"], built["col_rows"], O))


def test_without_tables_same_bits(layers):
    """A weight without segment tables (built per call in the workspace) gives the same bits."""
    L = layers["u3000x5000"]
    say("tiled with and without stored tables")
    built, W = device_layer(L, DEV)
    W0 = snk.SnackCOO(W.out_features, W.in_features, W.rows, W.cols, W.vals, W.row_offsets, W.col_perm,
                      W.col_rows, W.col_cols, W.col_offsets, blocks=None)
    assert W0.row_blocks is None and W.row_blocks is not None
    x_in, _ = acts(7700, 64, L["in_features"])
    X = to_device(x_in, DEV)
    b = torch.from_numpy(L["bias"]).to(DEV)
    assert torch.equal(snk.snack_coo_fwd(W, X, b), snk.snack_coo_fwd(W0, X, b))
    dy_in, _ = acts(7701, 64, L["out_features"])
    dY = to_device(dy_in, DEV)
    Wc, W0c = W.to_column_order(), W0.to_column_order()
    assert torch.equal(snk.snack_coo_bwd_input(Wc, dY), snk.snack_coo_bwd_input(W0c, dY))


def _dw(L, B, seed, bf16, mode, colorder=False):
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    if colorder:
        W = W.to_column_order()
    x_in, x64 = acts(seed, B, I, bf16)
    dy_in, dy64 = acts(seed + 1, B, O, bf16)
    X, dY = to_device(x_in, DEV, bf16), to_device(dy_in, DEV, bf16)
    with tile_mode(mode):
        dW = snk.snack_coo_grad_weight(W, X, dY)
    torch.cuda.synchronize()
    ref = oracle.grad_weight(O, I, built["rows"], built["cols"], x64, dy64, nthreads=NTHREADS)
    if colorder:
        ref = ref[built["col_perm"].astype(np.int64)]
    check_close(dW.cpu().numpy(), ref, B, f"dW mode={mode} col={colorder}")
    return dW


@pytest.mark.parametrize("name", ["u3000x5000", "e1100x7777", "d2000x4000", "u4000x600"])
def test_tiled_dw_b64(layers, name):
    say(f"tiled dW {name} B=64")
    _dw(layers[name], 64, 7800, False, None)


@pytest.mark.parametrize("B", [50, 128, 192])
def test_tiled_dw_batches(layers, B):
    say(f"tiled dW u3000x5000 B={B}")
    _dw(layers["u3000x5000"], B, 7900 + B, False, None)


def test_tiled_dw_bf16_and_column_order(layers):
    say("tiled dW bf16 / column-order values")
    _dw(layers["e1100x7777"], 64, 8000, True, None)
    _dw(layers["d2000x4000"], 64, 8010, False, None, colorder=True)


def test_tiled_dw_matches_untiled(layers):
    L = layers["d2000x4000"]
    say("tiled dW vs rowsddmm")
    a = _dw(L, 64, 8100, False, None)
    b = _dw(L, 64, 8100, False, "0")
    check_close(a.cpu().numpy(), b.cpu().numpy(), 64, "tiled vs rowsddmm dW")


def bwd_form(v):
    """snack_coo_bwd's form (SNACK_OPT_BWD_FORM): 'fused', 'split', 'tiled', or None for the library's choice."""
    return snk.option(snk.OPT_BWD_FORM, {None: -1, "fused": 0, "split": 1, "tiled": 2}[v])


@pytest.mark.parametrize("form", [None, "fused", "split", "tiled"])
@pytest.mark.parametrize("name,B", [("u3000x5000", 64), ("e1100x7777", 50), ("d2000x4000", 16),
                                    ("u4000x600", 32), ("u3000x5000", 128)])
def test_backward_forms(layers, name, B, form):
    """snack_coo_bwd in each form (one pass gathering dY from L2, two tiled passes, one tiled pass;
    a form that does not apply falls back to the library's choice), values in row and in column
    order: dX, dW (in the values' order) and db against the oracle."""
    L = layers[name]
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    assert nnz >= 1 << 20
    built, W = device_layer(L, DEV)
    x_in, x64 = acts(8200 + B, B, I)
    dy_in, dy64 = acts(8300 + B, B, O)
    X, dY = to_device(x_in, DEV), to_device(dy_in, DEV)
    r, c, v = built["rows"], built["cols"], built["vals"]
    dXr = oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS)
    dWr = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
    for order, w in (("row", W), ("col", W.to_column_order())):
        say(f"snack_coo_bwd {name} B={B} form={form} values in {order} order")
        db = torch.empty(O, dtype=torch.float32, device=DEV)
        with bwd_form(form):
            one_pass = snk.snack_coo_bwd_is_fused(w, B)
            dX, dW = snk.snack_coo_bwd(w, X, dY, db=db)
            torch.cuda.synchronize()
        if form in (None, "split") and order == "row" and B <= 64:
            assert not one_pass
        if form in ("fused", "tiled") or order == "col" or B > 64:
            assert one_pass
        ref_w = dWr[built["col_perm"].astype(np.int64)] if order == "col" else dWr
        check_close(dX.cpu().numpy(), dXr, nnz / I, f"bwd dX ({order})")
        check_close(dW.cpu().numpy(), ref_w, B, f"bwd dW ({order})")
        check_close(db.cpu().numpy(), oracle.grad_bias(dy64), B, f"bwd db ({order})")


@pytest.mark.parametrize("B", [512, 1024, 4096])
def test_tiled_large_batch(B):
    """Up to 64 batch tiles of 64 columns on the 5000 x 5000 layer at 90 % (the GAMLP shape): the
    forward, the input gradient (values through col_perm, gathered into walk order once), the
    weight gradient (batch tiles added in turn) and snack_coo_bwd against the oracle, in full."""
    spec, L = named_layer("gamlp90")
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    x_in, x64 = acts(8900 + B, B, I)
    dy_in, dy64 = acts(8950 + B, B, O)
    X, dY = to_device(x_in, DEV), to_device(dy_in, DEV)
    b = torch.from_numpy(L["bias"]).to(DEV)
    say(f"large batch B={B}")
    Y = snk.snack_coo_fwd(W, X, b)
    dX = snk.snack_coo_bwd_input(W, dY)
    dW = snk.snack_coo_grad_weight(W, X, dY)
    dX2, dW2 = snk.snack_coo_bwd(W, X, dY)
    torch.cuda.synchronize()
    r, c, v = built["rows"], built["cols"], built["vals"]
    check_close(Y.cpu().numpy(), oracle.fwd(O, I, r, c, v, x64, L["bias"], nthreads=NTHREADS), nnz / O, f"fwd B={B}")
    dXr = oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS)
    dWr = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
    check_close(dX.cpu().numpy(), dXr, nnz / I, f"dX B={B}")
    check_close(dW.cpu().numpy(), dWr, B, f"dW B={B}")
    check_close(dX2.cpu().numpy(), dXr, nnz / I, f"bwd dX B={B}")
    check_close(dW2.cpu().numpy(), dWr, B, f"bwd dW B={B}")


@pytest.mark.parametrize("B", [16, 32, 64])
@pytest.mark.parametrize("form", ["split", "tiled"])
def test_backward_forms_bf16(layers, form, B):
    """bf16 activations through the two-pass and one-pass tiled backward at one batch tile of 16,
    32 or 64 columns (dX rounded to bf16)."""
    L = layers["e1100x7777"]
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    x_in, x64 = acts(8400 + B, B, I, True)
    dy_in, dy64 = acts(8401 + B, B, O, True)
    X, dY = to_device(x_in, DEV, True), to_device(dy_in, DEV, True)
    r, c, v = built["rows"], built["cols"], built["vals"]
    for order, w in (("row", W), ("col", W.to_column_order())):
        say(f"snack_coo_bwd bf16 form={form} B={B} values in {order} order")
        with bwd_form(form):
            dX, dW = snk.snack_coo_bwd(w, X, dY)
            torch.cuda.synchronize()
        ref_w = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
        if order == "col":
            ref_w = ref_w[built["col_perm"].astype(np.int64)]
        check_close(from_device(dX), oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS), nnz / I,
                    f"bf16 bwd dX ({order})", True)
        check_close(dW.cpu().numpy(), ref_w, B, f"bf16 bwd dW ({order}) B={B}", True)


@pytest.mark.parametrize("order", ["row", "col"])
def test_tiled_backward_in_graph(layers, order):
    """The step with the tiled backward (two passes for row order, one for column order) captured
    in a HIP graph and replayed several times with eager work in between: every replay equals the
    eager result bit for bit."""
    L = layers["u3000x5000"]
    say(f"tiled step in a HIP graph, values in {order} order")
    built, W = device_layer(L, DEV)
    if order == "col":
        W = W.to_column_order()
    B = 64
    x_in, _ = acts(8500, B, L["in_features"])
    dy_in, _ = acts(8501, B, L["out_features"])
    X, dY = to_device(x_in, DEV), to_device(dy_in, DEV)
    b = torch.from_numpy(L["bias"]).to(DEV)
    need = max(snk.snack_coo_workspace_bytes(op, W, B, snk.SNACK_F32) for op in (0, 3))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    Y = torch.empty(B, L["out_features"], device=DEV)
    dX = torch.empty(B, L["in_features"], device=DEV)
    dW = torch.empty(L["nnz"], device=DEV)
    db = torch.empty(L["out_features"], device=DEV)

    def step():
        snk.snack_coo_fwd(W, X, b, out=Y, workspace=ws)
        snk.snack_coo_bwd(W, X, dY, dx_out=dX, dw_out=dW, db=db, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (Y, dX, dW, db)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for t in (Y, dX, dW, db):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((Y, dX, dW, db), ref):
            assert torch.equal(t, r)
        _ = X.sum()


def _tiled_random_cases(n=12, seed=5151):
    """Random layers of at least 2^20 entries (the tiled walks' threshold, which take them where
    their segments average 8 entries or more): shapes from a single
    column block to 15, four structures, padded and unpadded batches from 16 to 300 (one to five
    batch tiles of 64 columns, or tiles of 16 and 32), values in either order, a quarter bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = ["uniform", "empty_rows", "dense_lines", "skewed_rows"]
    batches = [16, 17, 32, 48, 64, 96, 100, 128, 192, 256, 300]
    out = []
    for i in range(n):
        O = int(rng.integers(600, 9000))
        I = int(rng.integers(600, 9000))
        B = batches[int(rng.integers(0, len(batches)))]
        nnz = int(min(O * I // 3, max(1 << 20, int(rng.uniform(1.05e6, 3.0e6))), 400_000_000 // B))
        shape = shapes[int(rng.integers(0, len(shapes)))]
        order = "col" if rng.random() < 0.5 else "row"
        bf16 = bool(rng.random() < 0.25)
        out.append((5200 + i, shape, O, I, nnz, B, order, bf16))
    return out


@pytest.mark.parametrize("case", _tiled_random_cases(),
                         ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-n{c[4]}-B{c[5]}-{c[6]}" + ("-bf16" if c[7] else ""))
def test_tiled_random_sweep(case):
    """Forward, input gradient, weight gradient and the backward call on random tiled layers
    against the oracle (per-feature reduction lengths in the bound); a second backward call gives
    the same bits."""
    seed, shape, O, I, nnz, B, order, bf16 = case
    say(f"tiled random {shape} {O}x{I} nnz={nnz} B={B} values in {order} order bf16={bf16}")
    L = synth.random_small_layer(seed, O, I, nnz, shape)
    assert L["nnz"] >= (1 << 20) or shape != "uniform"
    built, W = device_layer(L, DEV)
    if order == "col":
        W = W.to_column_order()
    nz = L["nnz"]
    x_in, x64 = acts(seed, B, I, bf16)
    dy_in, dy64 = acts(seed + 1, B, O, bf16)
    X, dY = to_device(x_in, DEV, bf16), to_device(dy_in, DEV, bf16)
    b = torch.from_numpy(L["bias"]).to(DEV)
    Y = snk.snack_coo_fwd(W, X, b)
    dX = snk.snack_coo_bwd_input(W, dY)
    dW = snk.snack_coo_grad_weight(W, X, dY)
    dX2, dW2 = snk.snack_coo_bwd(W, X, dY)
    dX3, dW3 = snk.snack_coo_bwd(W, X, dY)
    torch.cuda.synchronize()
    assert torch.equal(dX2, dX3) and torch.equal(dW2, dW3)
    r, c, v = built["rows"], built["cols"], built["vals"]
    check_close(from_device(Y), oracle.fwd(O, I, r, c, v, x64, L["bias"], nthreads=NTHREADS), row_counts(built),
                "fwd", bf16)
    dXr = oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS)
    check_close(from_device(dX), dXr, col_counts(built), "dX", bf16)
    check_close(from_device(dX2), dXr, col_counts(built), "bwd dX", bf16)
    dWr = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
    if order == "col":
        dWr = dWr[built["col_perm"].astype(np.int64)]
    check_close(dW.cpu().numpy(), dWr, B, "dW")
    check_close(dW2.cpu().numpy(), dWr, B, "bwd dW")
