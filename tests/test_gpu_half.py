"""The half-precision path (SNACK_BF16_HW: bf16 activations and bf16 weights, the forward and the
input gradient on gfx950's matrix cores over tiles of W made dense in LDS) against the fp64
oracle (needs a GPU).

The reference is the oracle run on the weights rounded to bf16 (nearest even, by the synthetic
data module's numpy conversion) and on the bf16 activations, so what is left is fp32
accumulation and the bf16 rounding of the outputs: every element within 2^-8 of its reference
magnitude plus the fp32 bound.  Against the oracle on the unrounded fp32 weights the outputs stay
within the bf16 variant's relative L2 of 1e-2 (no per-element bound: the weights' rounding adds
up over a key's entries).  The weight gradient does not read the weights and
is held to the bf16 tolerance as for SNACK_BF16.

Cases: several column blocks with a narrower last one, a single block (I = 600 < 638), full rows
and columns (segments of a whole block), empty rows, key counts that leave a partial last tile of
64 keys, batches of 1, 32, 64, 100, 130, 256, 300 and 512 (partial and several batch tiles, the
wide kernel's groups of four tiles with a partial last group), values in row order
and in column order (each kernel both with and without the value permutation), the 10000 x 10000
layer at 95 % and batch 64 in full, reruns equal bit for bit, the allocation-free forward equal to
the forward, and the shape and alignment errors of the path; and a seeded random sweep of 24 layers (feature
counts multiples of 8, six structures, batches 1 to 513, both value orders) through the forward,
the input gradient, the backward call and the matrix-core weight gradient.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import NTHREADS, acts, check_close, device_layer, from_device, named_layer, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import coo_spmm_row_amd as snk  # noqa: E402

DEV = torch.device("cuda:0")


def half(v):
    """The fp32 values rounded to bf16 (nearest even), as fp64."""
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(np.asarray(v, np.float32))).astype(np.float64)


def check_half(got, ref_half, ref_full, n_reduce, what):
    """got (bf16 outputs) against the oracle on bf16 weights, element by element, and against the
    oracle on the fp32 weights in relative L2."""
    got = np.asarray(got, np.float64)
    assert got.shape == ref_half.shape, f"{what}: shape {got.shape} vs {ref_half.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref_half)
    bound = 2.0 ** -8 * np.abs(ref_half) + 1e-4 * math.sqrt(max(1.0, n_reduce))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{what}: {len(bad)} elements off, first {tuple(bad[0])}: {got[tuple(bad[0])]} vs {ref_half[tuple(bad[0])]}"
    # against the fp32 weights only the bf16 variant's relative L2 applies: each weight's rounding
    # moves an output by up to 2^-9 of that product, which no per-element bound of the output's
    # own rounding covers on keys of thousands of entries
    rel = float(np.linalg.norm(got - ref_full)) / max(float(np.linalg.norm(ref_full)), 1e-30)
    assert rel <= 1e-2, f"{what} (fp32 weights): rel-L2 {rel:.3e} > 1e-2"


@pytest.fixture(scope="module")
def layers():
    return {
        # I = 5000: 8 blocks of 625 columns; O = 3000: 47 tiles of 64 keys, the last one of 56
        "u3000x5000": synth.random_small_layer(701, 3000, 5000, 1_200_000, "uniform"),
        # two full rows and two full columns: segments of a whole block
        "d2000x4000": synth.random_small_layer(703, 2000, 4000, 1_100_000, "dense_lines"),
        # I = 600 < one block; O = 4000: 7 blocks for the input gradient
        "u4000x600": synth.random_small_layer(704, 4000, 600, 1_050_000, "uniform"),
        # three in four rows empty
        "e1104x2048": synth.random_small_layer(705, 1104, 2048, 300_000, "empty_rows"),
    }


def _run(L, B, seed, order):
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    if order == "col":
        W = W.to_column_order()
    x_in, x64 = acts(seed, B, I, True)
    dy_in, dy64 = acts(seed + 1, B, O, True)
    X, dY = to_device(x_in, DEV, True), to_device(dy_in, DEV, True)
    b = torch.from_numpy(L["bias"]).to(DEV)
    Y = snk.snack_coo_fwd(W, X, b, half_weights=True)
    dX = snk.snack_coo_bwd_input(W, dY, half_weights=True)
    torch.cuda.synchronize()
    r, c, v = built["rows"], built["cols"], built["vals"]
    vh = half(v)
    check_half(from_device(Y), oracle.fwd(O, I, r, c, vh, x64, L["bias"], nthreads=NTHREADS),
               oracle.fwd(O, I, r, c, v, x64, L["bias"], nthreads=NTHREADS), nnz / O, f"half fwd ({order}) B={B}")
    check_half(from_device(dX), oracle.bwd_input(O, I, r, c, vh, dy64, nthreads=NTHREADS),
               oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS), nnz / I, f"half dX ({order}) B={B}")
    return W, X, dY, b, Y, dX, built, x64, dy64


@pytest.mark.parametrize("order", ["row", "col"])
@pytest.mark.parametrize("B", [1, 32, 64, 100, 130])
@pytest.mark.parametrize("name", ["u3000x5000", "d2000x4000", "u4000x600", "e1104x2048"])
def test_half_fwd_dx(layers, name, B, order):
    say(f"half-precision {name} B={B} values in {order} order")
    _run(layers[name], B, 9100 + B, order)


@pytest.mark.parametrize("order", ["row", "col"])
def test_half_bwd_rerun_and_db(layers, order):
    """snack_coo_bwd with half weights: dX as snack_coo_bwd_input, dW and db as for bf16
    activations; a second forward and input gradient equal the first bit for bit."""
    L = layers["u3000x5000"]
    O, I, nnz, B = L["out_features"], L["in_features"], L["nnz"], 64
    say(f"half-precision bwd and reruns, values in {order} order")
    W, X, dY, b, Y, dX, built, x64, dy64 = _run(L, B, 9300, order)
    db = torch.empty(O, device=DEV)
    dX2, dW2 = snk.snack_coo_bwd(W, X, dY, db=db, half_weights=True)
    Y2 = snk.snack_coo_fwd(W, X, b, half_weights=True)
    torch.cuda.synchronize()
    assert torch.equal(Y2, Y) and torch.equal(dX2, dX)
    r, c = built["rows"], built["cols"]
    dWr = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
    if order == "col":
        dWr = dWr[built["col_perm"].astype(np.int64)]
    check_close(dW2.cpu().numpy(), dWr, B, f"half bwd dW ({order})", True)
    check_close(db.cpu().numpy(), oracle.grad_bias(dy64), B, "half bwd db")


def test_half_target95_full():
    """The 10000 x 10000 layer at 95 % sparsity, batch 64, values in column order: forward, input
    gradient and the backward pass compared in full."""
    spec, L = named_layer("target95")
    say("half-precision target95 B=64")
    B = 64
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    W, X, dY, b, Y, dX, built, x64, dy64 = _run(L, B, 9400, "col")
    dX2, dW2 = snk.snack_coo_bwd(W, X, dY, half_weights=True)
    torch.cuda.synchronize()
    assert torch.equal(dX2, dX)
    dWr = oracle.grad_weight(O, I, built["rows"], built["cols"], x64, dy64, nthreads=NTHREADS)
    check_close(dW2.cpu().numpy(), dWr[built["col_perm"].astype(np.int64)], B, "half target95 dW", True)


def test_half_small_and_empty():
    """The 512 x 512 layer at batch 4 (one tile of keys, one of batch rows) and a layer with no
    entries (the forward gives the bias, the input gradient zeros)."""
    spec, L = named_layer("tiny")
    say("half-precision tiny B=4")
    _run(L, 4, 9500, "row")
    Le = synth.random_small_layer(706, 96, 64, 0, "uniform")
    built, W = device_layer(Le, DEV)
    x_in, _ = acts(9501, 8, 64, True)
    dy_in, _ = acts(9502, 8, 96, True)
    b = torch.from_numpy(Le["bias"]).to(DEV)
    Y = snk.snack_coo_fwd(W, to_device(x_in, DEV, True), b, half_weights=True)
    dX = snk.snack_coo_bwd_input(W, to_device(dy_in, DEV, True), half_weights=True)
    torch.cuda.synchronize()
    ref = np.broadcast_to(half(Le["bias"]), (8, 96))
    assert np.array_equal(from_device(Y), ref)
    assert not torch.any(dX.float() != 0)


def test_half_noalloc_equals_forward(layers):
    L = layers["u3000x5000"]
    say("half-precision allocation-free forward")
    built, W = device_layer(L, DEV)
    x_in, _ = acts(9600, 64, L["in_features"], True)
    X = to_device(x_in, DEV, True)
    b = torch.from_numpy(L["bias"]).to(DEV)
    Y = snk.snack_coo_fwd(W, X, b, half_weights=True)
    Y2 = torch.empty_like(Y)
    snk.snack_coo_fwd_noalloc(W, X, Y2, b, half_weights=True)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)


def test_half_shape_and_alignment_errors():
    """I not a multiple of 8, activations not 16-byte aligned, fp32 activations: errors before
    any launch."""
    L = synth.random_small_layer(707, 64, 100, 2000, "uniform")
    built, W = device_layer(L, DEV)
    X = torch.zeros(32, 100, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="multiple of 8"):
        snk.snack_coo_fwd(W, X, half_weights=True)
    L2 = synth.random_small_layer(708, 64, 96, 2000, "uniform")
    built2, W2 = device_layer(L2, DEV)
    base = torch.zeros(32 * 96 + 1, dtype=torch.bfloat16, device=DEV)
    Xm = base[1:].view(32, 96)  # 2-byte aligned
    with pytest.raises(RuntimeError, match="16-byte aligned"):
        snk.snack_coo_fwd(W2, Xm, half_weights=True)
    with pytest.raises(TypeError):
        snk.snack_coo_fwd(W2, torch.zeros(32, 96, device=DEV), half_weights=True)


@pytest.mark.parametrize("order", ["row", "col"])
def test_half_weights_layer(order):
    """SnackLinear(half_weights=True) on bf16 inputs of shape [2, 32, 1024]: Y and dX against the
    oracle on the bf16-rounded values, dW and db as for bf16 activations; the trainable values
    stay fp32."""
    from coo_spmm_row_amd.layer import SnackLinear
    say(f"SnackLinear half weights 1024->768 95% values in {order} order")
    layer = SnackLinear(1024, 768, sparsity=0.95, seed=13, device=DEV, value_order=order, half_weights=True)
    assert layer.vals.dtype == torch.float32
    I, O, n = 1024, 768, 64
    x_in, x64 = acts(9700, n, I, True)
    g_in, g64 = acts(9701, n, O, True)
    X = to_device(x_in, DEV, True).reshape(2, 32, I).requires_grad_(True)
    G = to_device(g_in, DEV, True).reshape(2, 32, O)
    Y = layer(X)
    (Y.float() * G.float()).sum().backward()
    torch.cuda.synchronize()
    r, c = layer.rows.cpu().numpy(), layer.cols.cpu().numpy()
    v = layer.vals.detach().cpu().numpy()
    if order == "col":  # values stored in column-view order: back to triple order for the oracle
        v = v[np.argsort(layer.col_perm.cpu().numpy())]
    b = layer.bias.detach().cpu().numpy()
    vh = half(v)
    nnz = layer.nnz
    check_half(from_device(Y.detach().reshape(n, O)), oracle.fwd(O, I, r, c, vh, x64, b, nthreads=NTHREADS),
               oracle.fwd(O, I, r, c, v, x64, b, nthreads=NTHREADS), nnz / O, f"layer half Y ({order})")
    check_half(from_device(X.grad.reshape(n, I)), oracle.bwd_input(O, I, r, c, vh, g64, nthreads=NTHREADS),
               oracle.bwd_input(O, I, r, c, v, g64, nthreads=NTHREADS), nnz / I, f"layer half dX ({order})")
    dWr = oracle.grad_weight(O, I, r, c, x64, g64, nthreads=NTHREADS)
    if order == "col":
        dWr = dWr[layer.col_perm.cpu().numpy().astype(np.int64)]
    check_close(layer.vals.grad.cpu().numpy(), dWr, n, f"layer half dW ({order})", True)
    check_close(layer.bias.grad.cpu().numpy(), oracle.grad_bias(g64), n, "layer half db")


@pytest.mark.parametrize("order", ["row", "col"])
@pytest.mark.parametrize("B", [256, 300, 512])
def test_half_wide_batches(layers, B, order):
    """Batches beyond one 64-column tile take the wide kernel (four batch tiles share each
    densified slab): one full group of four tiles, a second group with one partial tile (300), two
    groups (512)."""
    say(f"half-precision wide batches u3000x5000 B={B} values in {order} order")
    _run(layers["u3000x5000"], B, 9800 + B, order)


@pytest.mark.parametrize("B", [130, 300])
def test_half_short_keys_wide_batches(B):
    """Keys averaging under 64 entries stay on one batch tile per workgroup at any batch: the
    forward of this layer (39 entries per row) runs the per-tile kernel at B > 64, its input
    gradient (78 per column) the wide one."""
    L = synth.random_small_layer(709, 1536, 768, 60_000, "uniform")
    say(f"half-precision short keys s1536x768 B={B}")
    for order in ("row", "col"):
        _run(L, B, 9900 + B, order)


@pytest.mark.parametrize("order", ["row", "col"])
def test_half_wide_many_tiles(order):
    """The wide kernel over many tiles without K groups: an 8192 x 1024 layer at 10 % density and
    batch 1000 (forward: 128 key tiles x 4 batch groups, the last group partial, one K group; input
    gradient: 16 key tiles x 4 batch groups over 7 K groups, summed by the block sum)."""
    L = synth.random_small_layer(710, 8192, 1024, 838_861, "uniform")
    say(f"half-precision wide kernel s8192x1024 B=1000 values in {order} order")
    _run(L, 1000, 9950, order)


@pytest.mark.parametrize("B", [64, 300])
def test_half_graph_replays_match_eager(layers, B):
    """The half-precision forward, input gradient and backward (K groups with their block sum at
    batch 64, the wide kernel at 300) captured in a HIP graph and replayed four times with eager
    work in between: every replay equals the eager result bit for bit."""
    L = layers["u3000x5000"]
    say(f"half-precision graph replay B={B}")
    built, W = device_layer(L, DEV)
    W = W.to_column_order()
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    X = to_device(acts(9960, B, I, True)[0], DEV, True)
    dY = to_device(acts(9961, B, O, True)[0], DEV, True)
    bias = torch.from_numpy(L["bias"]).to(DEV)
    need = max(snk.snack_coo_workspace_bytes(op, W, B, snk.SNACK_BF16_HW) for op in (0, 1, 3))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    Y = torch.empty(B, O, dtype=torch.bfloat16, device=DEV)
    dX = torch.empty(B, I, dtype=torch.bfloat16, device=DEV)
    dX2 = torch.empty(B, I, dtype=torch.bfloat16, device=DEV)
    dW2 = torch.empty(nnz, device=DEV)
    db2 = torch.empty(O, device=DEV)
    outs = (Y, dX, dX2, dW2, db2)

    def step():
        snk.snack_coo_fwd(W, X, bias, out=Y, workspace=ws, half_weights=True)
        snk.snack_coo_bwd_input(W, dY, out=dX, workspace=ws, half_weights=True)
        snk.snack_coo_bwd(W, X, dY, dx_out=dX2, dw_out=dW2, db=db2, workspace=ws, half_weights=True)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), (rep, i)


@pytest.mark.parametrize("half_weights", [False, True], ids=["bf16", "bf16hw"])
@pytest.mark.parametrize("order", ["row", "col"])
@pytest.mark.parametrize("name,B", [("u3000x5000", 300), ("u3000x5000", 512), ("d2000x4000", 257),
                                    ("u4000x600", 384), ("e1104x2048", 1000)])
def test_bf16_weight_gradient_on_matrix_cores(layers, name, B, order, half_weights):
    """The weight gradient with bf16 activations at batches of 256 and more on the matrix cores
    (feature-major bf16 copies, dense 64 x 256 products over the batch sampled at the stored
    entries; forced by SNACK_OPT_BF16_DW_MFMA, which by default takes layers at least 1/12 dense),
    with fp32 or half weights alike: the products of bf16 values are exact in fp32, so it
    is held to the fp32 tolerance against the oracle on the same bf16 inputs, through
    snack_coo_grad_weight and snack_coo_bwd, in the values' order."""
    L = layers[name]
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    say(f"bf16 dW on the matrix cores {name} B={B} values in {order} order half_weights={half_weights}")
    built, W = device_layer(L, DEV)
    if order == "col":
        W = W.to_column_order()
    x_in, x64 = acts(9970 + B, B, I, True)
    dy_in, dy64 = acts(9971 + B, B, O, True)
    X, dY = to_device(x_in, DEV, True), to_device(dy_in, DEV, True)
    with snk.option(snk.OPT_BF16_DW_MFMA, 1):  # every layer here, dense enough or not
        dW = snk.snack_coo_grad_weight(W, X, dY, half_weights=half_weights)
        dX2, dW2 = snk.snack_coo_bwd(W, X, dY, half_weights=half_weights)
        torch.cuda.synchronize()
    ref = oracle.grad_weight(O, I, built["rows"], built["cols"], x64, dy64, nthreads=NTHREADS)
    if order == "col":
        ref = ref[built["col_perm"].astype(np.int64)]
    check_close(dW.cpu().numpy(), ref, B, f"bf16 dW {name} B={B} ({order})")
    check_close(dW2.cpu().numpy(), ref, B, f"bf16 bwd dW {name} B={B} ({order})")


def _half_random_cases(n=24, seed=8888):
    """Random layers whose feature counts are multiples of 8 (what the path requires), random
    densities and structures, batches from 1 to 513 (one partial tile, several tiles, the wide
    kernel's groups of four), values in either order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = ["uniform", "empty_rows", "dense_lines", "skewed_rows", "one_row", "one_col"]
    batches = [1, 3, 16, 33, 64, 65, 128, 255, 256, 300, 513]
    out = []
    for i in range(n):
        O = 8 * int(rng.integers(1, 400))
        I = 8 * int(rng.integers(1, 400))
        dens = float(10 ** rng.uniform(-3.0, -0.5))
        B = batches[int(rng.integers(0, len(batches)))]
        nnz = max(1, min(O * I, int(dens * O * I), 300_000_000 // B))
        shape = shapes[int(rng.integers(0, len(shapes)))]
        order = "col" if rng.random() < 0.5 else "row"
        out.append((9600 + i, shape, O, I, nnz, B, order))
    return out


@pytest.mark.parametrize("case", _half_random_cases(),
                         ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-n{c[4]}-B{c[5]}-{c[6]}")
def test_half_random_sweep(case):
    """Forward and input gradient with half weights against the oracle on the rounded weights
    (check_half), and the weight gradient of the same bf16 activations with the matrix-core form
    forced on at batches of 256 and more (fp32 tolerance), else the library's choice (bf16
    tolerance)."""
    seed, shape, O, I, nnz, B, order = case
    say(f"half random {shape} {O}x{I} nnz={nnz} B={B} values in {order} order")
    L = synth.random_small_layer(seed, O, I, nnz, shape)
    if L["nnz"] == 0:
        pytest.skip("the shape left no entries")
    W, X, dY, b, Y, dX, built, x64, dy64 = _run(L, B, seed, order)
    ref = oracle.grad_weight(O, I, built["rows"], built["cols"], x64, dy64, nthreads=NTHREADS)
    if order == "col":
        ref = ref[built["col_perm"].astype(np.int64)]
    if B >= 256:
        with snk.option(snk.OPT_BF16_DW_MFMA, 1):
            dW = snk.snack_coo_grad_weight(W, X, dY, half_weights=True)
            torch.cuda.synchronize()
        check_close(dW.cpu().numpy(), ref, B, f"half random dW (matrix cores) B={B}")
    dX2, dW2 = snk.snack_coo_bwd(W, X, dY, half_weights=True)
    torch.cuda.synchronize()
    assert torch.equal(dX2, dX)
    check_close(dW2.cpu().numpy(), ref, B, f"half random bwd dW B={B}", True)
