"""HIP path against the fp64 oracle, element by element, through the C ABI (needs a gfx950 GPU)."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (BANDINGS, NTHREADS, acts, band_threshold, check_close, col_counts, device_layer, from_device,
                      named_layer, row_counts, say, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import coo_spmm_row_amd as snk  # noqa: E402

DEV = torch.device("cuda:0")


def run_all(L, B, seed, bf16=False, bias=True):
    """fwd, dX, dW (+db) on the GPU and in the oracle; compare everything."""
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    x_in, x64 = acts(seed, B, I, bf16)
    dy_in, dy64 = acts(seed + 1, B, O, bf16)
    X, dY = to_device(x_in, DEV, bf16), to_device(dy_in, DEV, bf16)
    b = torch.from_numpy(L["bias"]).to(DEV) if bias else None
    Y = snk.snack_coo_fwd(W, X, b)
    db = torch.empty(O, dtype=torch.float32, device=DEV)
    dX = snk.snack_coo_bwd_input(W, dY, db=db)
    dW = snk.snack_coo_grad_weight(W, X, dY)
    torch.cuda.synchronize()
    r, c, v = built["rows"], built["cols"], built["vals"]
    Yr = oracle.fwd(O, I, r, c, v, x64, L["bias"] if bias else None, nthreads=NTHREADS)
    dXr = oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS)
    dWr = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
    check_close(from_device(Y), Yr, row_counts(built), "fwd", bf16)
    check_close(from_device(dX), dXr, col_counts(built), "dX", bf16)
    check_close(dW.cpu().numpy(), dWr, B, "dW")
    check_close(db.cpu().numpy(), oracle.grad_bias(dy64), B, "db")
    # both gradients from one call (one pass over the column view where the batch allows it)
    db2 = torch.empty(O, dtype=torch.float32, device=DEV)
    dX2, dW2 = snk.snack_coo_bwd(W, X, dY, db=db2)
    torch.cuda.synchronize()
    check_close(from_device(dX2), dXr, col_counts(built), "bwd dX", bf16)
    check_close(dW2.cpu().numpy(), dWr, B, "bwd dW")
    check_close(db2.cpu().numpy(), oracle.grad_bias(dy64), B, "bwd db")
    return built, W, X, dY, Y, dX, dW


# ------------------------------------------------------------ small shapes: tiles + ragged tails
SMALL = [  # seed, shape, O, I, nnz
    (101, "uniform", 300, 257, 9000),
    (102, "empty_rows", 129, 200, 3000),
    (103, "one_row", 50, 3000, 3000),
    (104, "one_col", 4000, 37, 4000),
    (105, "diag", 333, 333, 333),
    (106, "uniform", 1, 5000, 1500),
    (107, "uniform", 5000, 1, 700),
]
BATCHES = [1, 2, 3, 4, 5, 8, 12, 13, 16, 20, 24, 32, 48, 64, 68, 96, 100, 128, 130, 192]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}")
@pytest.mark.parametrize("B", BATCHES)
def test_small_shapes_fp32(case, B):
    seed, shape, O, I, nnz = case
    say(f"small fp32 {shape} {O}x{I} nnz={nnz} B={B}")
    L = synth.random_small_layer(seed, O, I, nnz, shape)
    run_all(L, B, seed + B)


@pytest.mark.parametrize("B", [1, 3, 4, 12, 16, 48, 64, 72])
def test_small_shapes_bf16(B):
    say(f"small bf16 B={B}")
    L = synth.random_small_layer(111, 260, 310, 8000, "empty_rows")
    run_all(L, B, 900 + B, bf16=True)


def test_no_bias_and_zero_batch():
    say("no bias, batch 0")
    L = synth.random_small_layer(121, 64, 80, 900, "uniform")
    run_all(L, 7, 5, bias=False)
    built, W = device_layer(L, DEV)
    X = torch.zeros((0, 80), device=DEV)
    assert snk.snack_coo_fwd(W, X).shape == (0, 64)
    dW = snk.snack_coo_grad_weight(W, X, torch.zeros((0, 64), device=DEV))
    torch.cuda.synchronize()
    assert not torch.any(dW)


def test_empty_layer():
    say("nnz = 0")
    L = {"rows": np.zeros(0, np.int32), "cols": np.zeros(0, np.int32), "vals": np.zeros(0, np.float32),
         "bias": np.linspace(-1, 1, 40).astype(np.float32), "out_features": 40, "in_features": 30, "nnz": 0}
    built, W = device_layer(L, DEV)
    for B in (1, 5, 64):
        X = torch.randn(B, 30, device=DEV)
        Y = snk.snack_coo_fwd(W, X, torch.from_numpy(L["bias"]).to(DEV))
        dX = snk.snack_coo_bwd_input(W, torch.randn(B, 40, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(Y, torch.from_numpy(L["bias"]).to(DEV).expand(B, 40))
        assert not torch.any(dX)


def test_long_rows_span_many_chunks():
    """A row far longer than one wave's chunk (power-law heavy rows)."""
    say("long rows")
    O, I = 6, 30000
    rng = np.random.Generator(np.random.PCG64(5))
    parts = []
    for r, n in ((1, 30000), (2, 1), (4, 17000)):
        parts.append(r * I + np.sort(rng.choice(I, n, replace=False)))
    pos = np.concatenate(parts)
    L = {"rows": (pos // I).astype(np.int32), "cols": (pos % I).astype(np.int32),
         "vals": rng.standard_normal(pos.size).astype(np.float32) * 0.01,
         "bias": rng.standard_normal(O).astype(np.float32), "out_features": O, "in_features": I, "nnz": pos.size}
    for B in (1, 2, 8, 16, 64):
        run_all(L, B, 40 + B)


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("B", [4])
def test_tiny_layer(B):
    say(f"tiny 512x512 90% B={B}")
    spec, L = named_layer("tiny")
    run_all(L, B, 1010)


@pytest.mark.parametrize("B", [1, 8, 32])
def test_mid_layer(B):
    say(f"mid 4096x4096 95% B={B}")
    spec, L = named_layer("mid")
    run_all(L, B, 2010 + B)


@pytest.mark.parametrize("name", ["xs99", "xs999", "xs99_zipf", "xs999_zipf"])
def test_extreme_sparse_batch1(name):
    say(f"{name} B=1")
    spec, L = named_layer(name)
    built, W, X, dY, Y, dX, dW = run_all(L, 1, 4010)
    # rows without entries output the bias exactly
    empty = np.flatnonzero(np.diff(built["row_offsets"]) == 0)
    if empty.size:
        assert np.array_equal(Y.cpu().numpy()[0, empty], L["bias"][empty])


@pytest.mark.parametrize("name", ["gamlp90", "gamlp95", "gamlp99"])
def test_gamlp_shaped_batch1(name):
    """The 5000 x 5000 GAMLP-shaped projection at batch 1 (all four products, full compare)."""
    say(f"{name} batch 1")
    spec, L = named_layer(name)
    run_all(L, 1, 7000 + spec.variant)


@pytest.mark.parametrize("name", ["gpt2_qkv", "gpt2_fc", "gpt2_proj"])
@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_gpt2_shapes(name, bf16):
    say(f"{name} B=1024 bf16={bf16}")
    spec, L = named_layer(name)
    run_all(L, 1024, 5010, bf16=bf16)


def _full_with_adjoint(name, B, seed):
    """Every output of the layer compared element by element with the oracle (run_all), then the
    adjoint identity <dY, Y - b> = <dX, X> = <dW, vals> on the full outputs in fp64."""
    spec, L = named_layer(name)
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W, X, dYt, Y, dX, dW = run_all(L, B, seed)
    x, _ = acts(seed, B, I)
    dy, _ = acts(seed + 1, B, O)
    Yb = Y.cpu().numpy().astype(np.float64) - L["bias"].astype(np.float64)
    a = float(np.sum(dy.astype(np.float64) * Yb))
    c = float(np.sum(dX.cpu().numpy().astype(np.float64) * x.astype(np.float64)))
    d = float(np.dot(dW.cpu().numpy().astype(np.float64), built["vals"].astype(np.float64)))
    scale = math.sqrt(B * O) * math.sqrt(nnz) * 1e-5 + 1e-3
    assert abs(a - c) <= scale and abs(a - d) <= scale, (a, c, d)


@pytest.mark.parametrize("B", [1, 16, 64])
def test_llm_scale_full_compare(B):
    say(f"llm90 10k 90% (10M entries) B={B} full compare")
    _full_with_adjoint("llm90", B, 3010 + B)


@pytest.mark.parametrize("B", [1, 64])
def test_target_layer_full_compare(B):
    say(f"target95 10k 95% B={B} full compare")
    _full_with_adjoint("target95", B, 3510 + B)


# ------------------------------------------------------------ invariants
def test_invariants_bias_determinism_scaling_permutation():
    say("invariants")
    L = synth.random_small_layer(131, 700, 900, 40000, "empty_rows")
    built, W = device_layer(L, DEV)
    b = torch.from_numpy(L["bias"]).to(DEV)
    for B in (1, 5, 64):
        X = to_device(synth.make_acts(77 + B, B, 900), DEV)
        dY = to_device(synth.make_acts(78 + B, B, 700), DEV)
        # X = 0 gives the bias exactly; dY = 0 gives dX = 0; X = 0 gives dW = 0
        assert torch.equal(snk.snack_coo_fwd(W, torch.zeros_like(X), b), b.expand(B, 700))
        assert not torch.any(snk.snack_coo_bwd_input(W, torch.zeros_like(dY)))
        assert not torch.any(snk.snack_coo_grad_weight(W, torch.zeros_like(X), dY))
        # deterministic: bit-identical reruns (below 2^21 entries the batch-1 input gradient walks
        # the column view, with no atomics)
        Y1, Y2 = snk.snack_coo_fwd(W, X, b), snk.snack_coo_fwd(W, X, b)
        assert torch.equal(Y1, Y2)
        dX1, dX2 = snk.snack_coo_bwd_input(W, dY), snk.snack_coo_bwd_input(W, dY)
        assert torch.equal(dX1, dX2)
        assert torch.equal(snk.snack_coo_grad_weight(W, X, dY), snk.snack_coo_grad_weight(W, X, dY))
        if 2 <= B <= 256:  # the fused backward pass has no atomics: bit-identical reruns
            a, b2 = snk.snack_coo_bwd(W, X, dY), snk.snack_coo_bwd(W, X, dY)
            assert torch.equal(a[0], b2[0]) and torch.equal(a[1], b2[1])
        # power-of-two scaling is exact
        assert torch.equal(snk.snack_coo_fwd(W, 2 * X), 2 * snk.snack_coo_fwd(W, X))
        # empty rows output the bias exactly
        empty = torch.from_numpy(np.flatnonzero(np.diff(built["row_offsets"]) == 0)).to(DEV)
        assert empty.numel() > 0
        assert torch.equal(Y1[:, empty], b[empty].expand(B, -1))
        # a permuted input order builds the same layer and the same outputs
        p = np.random.Generator(np.random.PCG64(B)).permutation(L["nnz"])
        built2 = snk.snack_coo_build(700, 900, L["rows"][p], L["cols"][p], L["vals"][p])
        W2 = snk.SnackCOO.from_built(built2, DEV)
        assert torch.equal(snk.snack_coo_fwd(W2, X, b), Y1)
    # true sparsity: device bytes of the weight are 12 nnz + 4 (O+1) plus the column view
    nnz, O, I = L["nnz"], 700, 900
    assert W.device_bytes(blocks=False) == 12 * nnz + 4 * (O + 1) + 12 * nnz + 4 * (I + 1)
    # plus the segment lists of the tiled kernels: a 16-byte record per (row, block) and per
    # (column, block)
    nb_r, nb_c = -(-I // 638), -(-O // 638)
    assert W.device_bytes() == W.device_bytes(blocks=False) + 16 * (O * nb_r + I * nb_c)


def test_linearity_in_x():
    say("linearity")
    L = synth.random_small_layer(141, 300, 400, 12000, "uniform")
    built, W = device_layer(L, DEV)
    X1 = to_device(synth.make_acts(1, 16, 400), DEV)
    X2 = to_device(synth.make_acts(2, 16, 400), DEV)
    lhs = snk.snack_coo_fwd(W, 0.5 * X1 - 3.0 * X2).cpu().numpy().astype(np.float64)
    rhs = 0.5 * snk.snack_coo_fwd(W, X1).cpu().numpy().astype(np.float64) - \
        3.0 * snk.snack_coo_fwd(W, X2).cpu().numpy().astype(np.float64)
    check_close(lhs, rhs, 40, "linearity")


def test_single_entry_and_stored_zero():
    say("single entry / stored zero")
    L = {"rows": np.array([3], np.int32), "cols": np.array([5], np.int32), "vals": np.array([0.0], np.float32),
         "bias": np.arange(8, dtype=np.float32), "out_features": 8, "in_features": 9, "nnz": 1}
    built, W = device_layer(L, DEV)
    X = to_device(synth.make_acts(3, 4, 9), DEV)
    dY = to_device(synth.make_acts(4, 4, 8), DEV)
    dW = snk.snack_coo_grad_weight(W, X, dY).cpu().numpy()
    ref = float(np.dot(dY.cpu().numpy()[:, 3].astype(np.float64), X.cpu().numpy()[:, 5].astype(np.float64)))
    assert dW.shape == (1,) and abs(dW[0] - ref) <= 1e-5 * (1 + abs(ref))  # a stored zero still gets its gradient


def test_workspace_contract():
    say("workspace")
    L = synth.random_small_layer(151, 100, 120, 2000, "uniform")
    built, W = device_layer(L, DEV)
    X = to_device(synth.make_acts(5, 8, 120), DEV)
    need = snk.snack_coo_workspace_bytes(snk.OP_FWD, W, 8, snk.SNACK_F32)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_fwd(W, X, workspace=small)
    assert e.value.status == "WORKSPACE"
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    assert torch.equal(snk.snack_coo_fwd(W, X, workspace=ws), snk.snack_coo_fwd(W, X))


# Larger layers at batches 64 / 128 / 192: ragged tiles, odd shapes, 600 to 20000 keys, full rows
# and columns (keys with thousands of entries next to keys with a few), rows with no entries
# (three in four), and the column permutation of the input gradient.
WIDE = [  # seed, shape, O, I, density
    (191, "uniform", 3000, 1300, 0.05),
    (192, "dense_lines", 2600, 2100, 0.06),
    (193, "uniform", 20000, 600, 0.05),
    (194, "uniform", 600, 20000, 0.05),
    (195, "uniform", 1100, 700, 0.10),
    (197, "empty_rows", 4000, 1300, 0.05),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}")
@pytest.mark.parametrize("B", [1, 64, 128])
def test_wide_layer_shapes(case, B):
    seed, shape, O, I, density = case
    say(f"wide layer {shape} {O}x{I} B={B}")
    L = synth.random_small_layer(seed, O, I, int(density * O * I), shape)
    run_all(L, B, 77 + B)


# Batch 1 on layers of more than 2M entries with up to 10240 columns and rows of hundreds to
# thousands of entries: the streamed row-order kernels for all three products (the input
# gradient with per-wave private copies), with full rows and columns, and three rows in four
# empty.
BATCH1_LARGE = [  # seed, shape, O, I, density
    (198, "dense_lines", 2500, 10000, 0.09),
    (199, "empty_rows", 4000, 9000, 0.06),
]


@pytest.mark.parametrize("case", BATCH1_LARGE, ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}")
@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_batch1_large_layers(case, bf16):
    seed, shape, O, I, density = case
    say(f"batch-1 large {shape} {O}x{I} bf16={bf16}")
    L = synth.random_small_layer(seed, O, I, int(density * O * I), shape)
    assert L["nnz"] >= 2 ** 21
    run_all(L, 1, 500 + seed, bf16=bf16)


def _check_bwd(L, B, seed, bf16=False):
    """snack_coo_bwd (dX, dW, db) against the oracle."""
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    x_in, x64 = acts(seed, B, I, bf16)
    dy_in, dy64 = acts(seed + 1, B, O, bf16)
    X, dY = to_device(x_in, DEV, bf16), to_device(dy_in, DEV, bf16)
    db = torch.empty(O, dtype=torch.float32, device=DEV)
    dX, dW = snk.snack_coo_bwd(W, X, dY, db=db)
    torch.cuda.synchronize()
    r, c, v = built["rows"], built["cols"], built["vals"]
    check_close(from_device(dX), oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS), col_counts(built), "dX",
                bf16)
    check_close(dW.cpu().numpy(), oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS), B, "dW")
    check_close(db.cpu().numpy(), oracle.grad_bias(dy64), B, "db")
    # a second call gives the same bits (fixed summation order, band partials added in order)
    dX2, dW2 = snk.snack_coo_bwd(W, X, dY)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX2) and torch.equal(dW, dW2)


def test_batch1_input_gradient_misaligned_arrays():
    """cols and vals 4 bytes off a 16-byte boundary: the batch-1 input gradient cannot take its
    16-byte loads and runs another kernel; the result must still match the oracle."""
    seed, shape, O, I, density = BATCH1_LARGE[1]
    say(f"batch-1 input gradient, misaligned cols/vals, {shape} {O}x{I}")
    L = synth.random_small_layer(seed, O, I, int(density * O * I), shape)
    built, W = device_layer(L, DEV)
    nnz = L["nnz"]
    cols = torch.empty(nnz + 1, dtype=torch.int32, device=DEV)[1:]
    vals = torch.empty(nnz + 1, dtype=torch.float32, device=DEV)[1:]
    cols.copy_(W.cols)
    vals.copy_(W.vals)
    assert cols.data_ptr() % 16 and vals.data_ptr() % 16
    Wm = snk.SnackCOO(O, I, W.rows, cols, vals, W.row_offsets, W.col_perm, W.col_rows, W.col_cols, W.col_offsets)
    assert snk._lib.snack_coo_workspace_bytes(snk.OP_BWD_INPUT, Wm.desc, 1, 0) > 0
    dy_in, dy64 = acts(1700, 1, O)
    dY = to_device(dy_in, DEV)
    dX = snk.snack_coo_bwd_input(Wm, dY)
    dXa = snk.snack_coo_bwd_input(W, dY)
    torch.cuda.synchronize()
    ref = oracle.bwd_input(O, I, built["rows"], built["cols"], built["vals"], dy64, nthreads=NTHREADS)
    check_close(from_device(dX), ref, nnz / I, "dX misaligned")
    check_close(from_device(dXa), ref, nnz / I, "dX aligned")


# snack_coo_bwd over batches that pick each variant of the one-pass backward (the batch padded
# with zero columns to Bp = 4*BT*Q, BT the largest power of two <= 16 leaving Q <= 4: 4 -> BT 1,
# 8 -> BT 2, 12 -> BT 1 Q 3, 16 -> BT 4, 24 -> BT 2 Q 3, 32 -> BT 8, 48 -> BT 4 Q 3,
# 64/128/192/256 -> BT 16 with Q 1..4; padded: 5 -> 8, 13 -> 16, 20 -> 24, 40 -> 48, 65 -> 96,
# 130 -> 192, 200 -> 256) and a batch that runs the two separate calls (512); fp32 and bf16; the
# one-pass kernel with and without row bands.
@pytest.mark.parametrize("banding", list(BANDINGS))
@pytest.mark.parametrize("B", [4, 5, 8, 12, 13, 16, 20, 24, 32, 40, 48, 64, 65, 96, 128, 130, 192, 200, 256, 512])
@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_backward_batches(B, bf16, banding):
    say(f"backward B={B} bf16={bf16} {banding}")
    L = synth.random_small_layer(181, 700, 900, 60000, "dense_lines")
    with band_threshold(BANDINGS[banding]):
        _check_bwd(L, B, 40 + B, bf16)


# The row-banded backward on layers whose bands are uneven or empty: rows holding more than an
# eighth of the entries (several band boundaries fall on one row), three rows in four empty, full
# rows and columns, rows skewed so that neither the band rows nor the columns' band ranges are
# where a uniform guess puts them (the full searches run), columns longer and shorter than a
# wave, and layers of 1 row or 1 column.
BANDED = [  # seed, shape, O, I, nnz
    (211, "one_row", 40, 5000, 5000),
    (212, "empty_rows", 3000, 900, 120000),
    (213, "dense_lines", 2600, 2100, 300000),
    (214, "uniform", 9000, 300, 400000),
    (215, "uniform", 300, 9000, 200000),
    (216, "uniform", 1, 5000, 1500),
    (217, "uniform", 5000, 1, 700),
    (218, "diag", 333, 333, 333),
    (219, "dense_lines", 50, 20000, 50000),
    (220, "skewed_rows", 4000, 1200, 400000),
]


@pytest.mark.parametrize("case", BANDED, ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}")
@pytest.mark.parametrize("B", [3, 4, 8, 16, 48, 64, 65, 128])
def test_backward_row_bands(case, B):
    seed, shape, O, I, nnz = case
    say(f"banded backward {shape} {O}x{I} nnz={nnz} B={B}")
    L = synth.random_small_layer(seed, O, I, nnz, shape)
    with band_threshold(1):
        _check_bwd(L, B, 900 + seed + B)


# Wide batches on a layer of more than 2^18 entries: the input gradient gathers the values into
# column order first (4+ batch tiles) and the weight gradient runs in 256-column slices that add
# into dW (B = 512: 2 slices, 1024: 4); full rows and columns included.
@pytest.mark.parametrize("B,bf16", [(256, False), (512, False), (1024, False), (512, True)],
                         ids=["B256", "B512", "B1024", "B512-bf16"])
def test_wide_batch_large_layer(B, bf16):
    say(f"wide batch B={B} bf16={bf16} on 1500x2000 10%")
    L = synth.random_small_layer(230, 1500, 2000, 300000, "dense_lines")
    assert L["nnz"] >= 2 ** 18
    run_all(L, B, 800 + B, bf16=bf16)


@pytest.mark.parametrize("B", [64, 192])
def test_wide_layer_bf16(B):
    say(f"wide layer bf16 B={B}")
    L = synth.random_small_layer(196, 2600, 2100, int(0.06 * 2600 * 2100), "dense_lines")
    run_all(L, B, 300 + B, bf16=True)


# ------------------------------------------------------------ seeded random sweep
def _random_cases(n=36, seed=4242):
    """Random shapes, densities, structures and batches (including 1, odd sizes, 16..192 and a
    few wide ones); each is checked in full by run_all (forward, both gradients separately and
    in one call, bias gradient)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = ["uniform", "empty_rows", "dense_lines", "skewed_rows", "one_row", "one_col"]
    batches = [1, 2, 3, 4, 5, 7, 8, 12, 16, 20, 24, 32, 36, 48, 64, 96, 128, 132, 192, 256, 320]
    out = []
    for i in range(n):
        O = int(rng.integers(1, 2500))
        I = int(rng.integers(1, 2500))
        dens = float(10 ** rng.uniform(-3.0, -0.7))
        nnz = max(1, min(O * I, int(dens * O * I)))
        shape = shapes[int(rng.integers(0, len(shapes)))]
        B = batches[int(rng.integers(0, len(batches)))]
        bf16 = bool(rng.random() < 0.25)
        out.append((5000 + i, shape, O, I, nnz, B, bf16))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-n{c[4]}-B{c[5]}"
                         + ("-bf16" if c[6] else ""))
def test_random_sweep(case):
    seed, shape, O, I, nnz, B, bf16 = case
    say(f"random {shape} {O}x{I} nnz={nnz} B={B} bf16={bf16}")
    L = synth.random_small_layer(seed, O, I, nnz, shape)
    if L["nnz"] == 0:
        pytest.skip("the shape left no entries")
    run_all(L, B, seed, bf16=bf16)


@pytest.mark.parametrize("B", [512, 1024])
@pytest.mark.parametrize("order", ["row", "col"])
@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_backward_shared_copies_equal_separate_calls(bf16, order, B):
    """snack_coo_bwd on an untiled layer at a wide batch, where both gradients take the row-wave
    kernels and the feature-major copies of X and dY are made once for both (a GPT-2-shaped
    768 -> 3072 layer at 1 % density), equals snack_coo_bwd_input and snack_coo_grad_weight
    called separately, bit for bit (the same kernels on the same copies), and the oracle; values
    in row order and in column order."""
    say(f"shared-copy backward B={B} bf16={bf16} values in {order} order")
    L = synth.random_small_layer(231, 3072, 768, 23593, "uniform")
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    if order == "col":
        W = W.to_column_order()
    assert snk.snack_coo_bwd_is_fused(W, B, snk.SNACK_BF16 if bf16 else snk.SNACK_F32) == 0
    x_in, x64 = acts(2300 + B, B, I, bf16)
    dy_in, dy64 = acts(2301 + B, B, O, bf16)
    X, dY = to_device(x_in, DEV, bf16), to_device(dy_in, DEV, bf16)
    db = torch.empty(O, dtype=torch.float32, device=DEV)
    dX, dW = snk.snack_coo_bwd(W, X, dY, db=db)
    dXs = snk.snack_coo_bwd_input(W, dY)
    dWs = snk.snack_coo_grad_weight(W, X, dY)
    torch.cuda.synchronize()
    assert torch.equal(dX, dXs) and torch.equal(dW, dWs)
    r, c, v = built["rows"], built["cols"], built["vals"]
    check_close(from_device(dX), oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS), nnz / I, "dX", bf16)
    dWr = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
    if order == "col":
        dWr = dWr[built["col_perm"].astype(np.int64)]
    check_close(dW.cpu().numpy(), dWr, B, "dW")
    check_close(db.cpu().numpy(), oracle.grad_bias(dy64), B, "db")
