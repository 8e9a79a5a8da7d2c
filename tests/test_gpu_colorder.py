"""Values kept in column-view order (snack_coo_desc.row_to_col) against the oracle and against the
same weight with values in row order (needs a GPU).

With the values in column order every product is the same; vals and every dW are stored in
column-view order (dW[j] belongs to triple entry col_perm[j]).  The forward walks the same rows in
the same order and the weight-gradient kernels compute the same per-entry sums, so Y and dW must
equal the row-order results bit for bit (dW permuted) -- Y except on untiled layers whose rows
average 256 entries or more at batches of 4 and more, where the row-order walk splits each row over
four waves; dX is checked against the oracle (the column walk may split long columns over four
waves when no permutation is read, and the fused pass drops its row bands, both of which change
the summation order only).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import NTHREADS, acts, check_close, col_counts, device_layer, from_device, row_counts, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import coo_spmm_row_amd as snk  # noqa: E402

DEV = torch.device("cuda:0")


def _run(L, B, seed, bf16=False):
    O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
    built, W = device_layer(L, DEV)
    Wc = W.to_column_order()
    assert Wc.column_order and not W.column_order
    cp = built["col_perm"].astype(np.int64)
    x_in, x64 = acts(seed, B, I, bf16)
    dy_in, dy64 = acts(seed + 1, B, O, bf16)
    X, dY = to_device(x_in, DEV, bf16), to_device(dy_in, DEV, bf16)
    b = torch.from_numpy(L["bias"]).to(DEV)
    out = {}
    for tag, w in (("row", W), ("col", Wc)):
        db = torch.empty(O, dtype=torch.float32, device=DEV)
        db2 = torch.empty(O, dtype=torch.float32, device=DEV)
        out[tag] = dict(Y=snk.snack_coo_fwd(w, X, b), dX=snk.snack_coo_bwd_input(w, dY, db=db),
                        dW=snk.snack_coo_grad_weight(w, X, dY), db=db)
        out[tag]["bdX"], out[tag]["bdW"] = snk.snack_coo_bwd(w, X, dY, db=db2)
        out[tag]["bdb"] = db2
    torch.cuda.synchronize()
    r, c, v = built["rows"], built["cols"], built["vals"]
    dXr = oracle.bwd_input(O, I, r, c, v, dy64, nthreads=NTHREADS)
    dWr = oracle.grad_weight(O, I, r, c, x64, dy64, nthreads=NTHREADS)
    R, C = out["row"], out["col"]
    # Y and dW: bit for bit the row-order results (dW in column order); Y only where both walks sum
    # each row in one order: the untiled row-order forward splits rows averaging 256 entries or more
    # over four waves, the column-order one (values through row_to_col) does not
    if nnz < 256 * O or nnz >= (1 << 20) or B < 4:
        assert torch.equal(R["Y"], C["Y"]), "Y differs"
    assert np.array_equal(C["dW"].cpu().numpy().view(np.uint32), R["dW"].cpu().numpy()[cp].view(np.uint32))
    assert np.array_equal(C["bdW"].cpu().numpy().view(np.uint32), R["bdW"].cpu().numpy()[cp].view(np.uint32))
    # against the oracle
    check_close(from_device(C["Y"]), oracle.fwd(O, I, r, c, v, x64, L["bias"], nthreads=NTHREADS),
                row_counts(built), "col Y", bf16)
    check_close(from_device(C["dX"]), dXr, col_counts(built), "col dX", bf16)
    check_close(from_device(C["bdX"]), dXr, col_counts(built), "col bwd dX", bf16)
    check_close(C["dW"].cpu().numpy(), dWr[cp], B, "col dW")
    check_close(C["bdW"].cpu().numpy(), dWr[cp], B, "col bwd dW")
    for k in ("db", "bdb"):
        check_close(C[k].cpu().numpy(), oracle.grad_bias(dy64), B, f"col {k}")
    return built, W, Wc


SHAPES = [  # seed, shape, O, I, nnz
    (301, "uniform", 300, 257, 9000),
    (302, "empty_rows", 129, 200, 3000),
    (303, "one_row", 50, 3000, 3000),
    (304, "one_col", 4000, 37, 4000),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}")
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 12, 16, 20, 48, 64, 130])
def test_column_order_small(case, B):
    seed, shape, O, I, nnz = case
    say(f"column-order values {shape} {O}x{I} B={B}")
    _run(synth.random_small_layer(seed, O, I, nnz, shape), B, seed + B)


@pytest.mark.parametrize("B", [1, 4, 16, 64])
def test_column_order_bf16(B):
    say(f"column-order values bf16 B={B}")
    _run(synth.random_small_layer(311, 260, 310, 8000, "empty_rows"), B, 950 + B, bf16=True)


@pytest.mark.parametrize("B", [1, 16, 64, 256, 512])
def test_column_order_large_layer(B):
    """1500 x 2000 at 10 % (300,000 entries): the forward reads through row_to_col with 4 batch tiles
    (B = 256: the values are gathered into row order first), 256-column slices of the weight
    gradient (B = 512), batch-1 kernels on gathered values."""
    say(f"column-order values 1500x2000 B={B}")
    _run(synth.random_small_layer(312, 1500, 2000, 300000, "dense_lines"), B, 1200 + B)


def test_column_order_batch1_private_copies():
    """A layer of more than 2^21 entries at batch 1 (the private-copy input gradient)."""
    say("column-order values batch 1, 2500x10000 9%")
    _run(synth.random_small_layer(313, 2500, 10000, 2250000, "dense_lines"), 1, 1300)


def test_conversions_and_topology_refusal():
    say("column-order conversions")
    L = synth.random_small_layer(314, 700, 900, 60000, "uniform")
    built, W = device_layer(L, DEV)
    Wc = W.to_column_order()
    cp = built["col_perm"]
    inv = np.empty_like(cp)
    inv[cp] = np.arange(cp.size, dtype=np.int32)
    assert np.array_equal(Wc.row_to_col.cpu().numpy(), inv)
    assert np.array_equal(Wc.vals.cpu().numpy().view(np.uint32), built["vals"][cp].view(np.uint32))
    back = Wc.to_row_order()
    assert not back.column_order
    assert np.array_equal(back.vals.cpu().numpy().view(np.uint32), built["vals"].view(np.uint32))
    assert Wc.to_column_order() is Wc and W.to_row_order() is W
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_topology_update_device(Wc, 10, 1)
    assert e.value.status == "UNSORTED"
    # in-place value updates keep working through the descriptor
    Wc.vals.mul_(2.0)
    X = torch.randn(8, 900, device=DEV)
    assert torch.equal(snk.snack_coo_fwd(Wc, X), snk.snack_coo_fwd(W, X * 2.0))


def _random_cases(n=24, seed=7373):
    """Random shapes, densities, structures and batches (1 to 1024: one-pass, two-pass and shared-copy
    backward forms, batch slices of the weight gradient), a quarter in bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = ["uniform", "empty_rows", "dense_lines", "skewed_rows", "one_row", "one_col"]
    batches = [1, 3, 4, 12, 16, 32, 48, 64, 65, 128, 256, 512, 1024]
    out = []
    for i in range(n):
        O = int(rng.integers(1, 3000))
        I = int(rng.integers(1, 3000))
        dens = float(10 ** rng.uniform(-3.0, -0.7))
        B = batches[int(rng.integers(0, len(batches)))]
        nnz = max(1, min(O * I, int(dens * O * I), 300_000_000 // B))
        shape = shapes[int(rng.integers(0, len(shapes)))]
        bf16 = bool(rng.random() < 0.25)
        out.append((7400 + i, shape, O, I, nnz, B, bf16))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-n{c[4]}-B{c[5]}"
                         + ("-bf16" if c[6] else ""))
def test_column_order_random_sweep(case):
    seed, shape, O, I, nnz, B, bf16 = case
    say(f"column order random {shape} {O}x{I} nnz={nnz} B={B} bf16={bf16}")
    L = synth.random_small_layer(seed, O, I, nnz, shape)
    if L["nnz"] == 0:
        pytest.skip("the shape left no entries")
    _run(L, B, seed, bf16)
