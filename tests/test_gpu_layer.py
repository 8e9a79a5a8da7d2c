"""SnackLinear (nn.Module + autograd.Function over the C ABI) against the fp64 oracle (needs a GPU)."""
import numpy as np
import pytest

import oracle
from gpu_util import NTHREADS, acts, check_close, from_device, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from coo_spmm_row_amd.layer import SnackLinear  # noqa: E402

DEV = torch.device("cuda:0")


def _host(layer):
    return (layer.rows.cpu().numpy(), layer.cols.cpu().numpy(), layer.vals.detach().cpu().numpy(),
            None if layer.bias is None else layer.bias.detach().cpu().numpy())


def _run(layer, lead, seed, bf16=False, x_grad=True):
    """Forward on X of shape lead + [I] and backward of sum(Y * G); returns host copies and the
    oracle's Y, dX, dW, db for the flattened batch."""
    I, O = layer.in_features, layer.out_features
    n = int(np.prod(lead))
    x_in, x64 = acts(seed, n, I, bf16)
    g_in, g64 = acts(seed + 1, n, O, bf16)
    X = to_device(x_in, DEV, bf16).reshape(*lead, I)
    G = to_device(g_in, DEV, bf16).reshape(*lead, O)
    X.requires_grad_(x_grad)
    Y = layer(X)
    assert Y.shape == (*lead, O) and Y.dtype == X.dtype
    (Y.float() * G.float()).sum().backward()  # dL/dY = G (exactly representable in X's dtype)
    torch.cuda.synchronize()
    r, c, v, b = _host(layer)
    ref = {"Y": oracle.fwd(O, I, r, c, v, x64, b, nthreads=NTHREADS),
           "dX": oracle.bwd_input(O, I, r, c, v, g64, nthreads=NTHREADS),
           "dW": oracle.grad_weight(O, I, r, c, x64, g64, nthreads=NTHREADS),
           "db": oracle.grad_bias(g64)}
    return X, Y, ref


@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
@pytest.mark.parametrize("lead", [(4,), (2, 3, 16), (64,)], ids=["B4", "B2x3x16", "B64"])
def test_layer_matches_oracle(lead, bf16):
    say(f"SnackLinear 300->200 90% lead={lead} bf16={bf16}")
    layer = SnackLinear(300, 200, sparsity=0.9, seed=11).to(DEV)
    X, Y, ref = _run(layer, lead, 500 + len(lead), bf16)
    n = int(np.prod(lead))
    nnz = layer.nnz
    check_close(from_device(Y.detach().reshape(n, 200)), ref["Y"], nnz / 200, "layer Y", bf16)
    check_close(from_device(X.grad.reshape(n, 300)), ref["dX"], nnz / 300, "layer dX", bf16)
    check_close(layer.vals.grad.cpu().numpy(), ref["dW"], n, "layer dW")
    check_close(layer.bias.grad.cpu().numpy(), ref["db"], n, "layer db")


def test_layer_grads_accumulate_and_partial_needs():
    say("SnackLinear gradient accumulation, frozen input / frozen values / no bias")
    layer = SnackLinear(257, 130, sparsity=0.8, seed=12).to(DEV)
    X, Y, ref = _run(layer, (16,), 600)
    g1 = (X.grad.clone(), layer.vals.grad.clone(), layer.bias.grad.clone())
    layer(X).sum().mul(0).backward()  # adds zero: grads unchanged
    (layer(X) * 0).sum().backward()
    assert torch.equal(layer.vals.grad, g1[1]) and torch.equal(layer.bias.grad, g1[2])
    # a second identical backward doubles every gradient exactly
    Gt = torch.from_numpy(acts(601, 16, 130)[0]).to(DEV)
    (layer(X) * Gt).sum().backward()
    assert torch.equal(layer.vals.grad, 2 * g1[1]) and torch.equal(layer.bias.grad, 2 * g1[2])
    assert torch.equal(X.grad, 2 * g1[0])
    # input without grad: weight and bias gradients only
    layer.zero_grad(set_to_none=True)
    X2 = X.detach()
    (layer(X2) * Gt).sum().backward()
    assert torch.equal(layer.vals.grad, g1[1]) and torch.equal(layer.bias.grad, g1[2])
    # frozen values: input and bias gradients only (the input gradient then comes from the
    # separate SpMM over the column view: equal to rounding, not bit for bit)
    layer.zero_grad(set_to_none=True)
    layer.vals.requires_grad_(False)
    X3 = X.detach().requires_grad_(True)
    (layer(X3) * Gt).sum().backward()
    assert layer.vals.grad is None
    check_close(X3.grad.cpu().numpy(), ref["dX"], layer.nnz / 257, "frozen-values dX")
    assert torch.equal(layer.bias.grad, g1[2])
    # no bias: the output is the pure SpMM
    nb = SnackLinear(257, 130, sparsity=0.8, seed=12, bias=False).to(DEV)
    r, c, v, _ = _host(nb)
    Y = nb(X.detach())
    check_close(Y.detach().cpu().numpy(), oracle.fwd(130, 257, r, c, v, X.detach().cpu().numpy().astype(np.float64),
                                                     None, nthreads=NTHREADS), nb.nnz / 130, "no-bias Y")


def test_layer_prune_and_regrow_then_train():
    say("SnackLinear prune-and-regrow, then forward/backward on the new support")
    layer = SnackLinear(400, 300, sparsity=0.95, seed=13).to(DEV)
    r, c, v, _ = _host(layer)
    trials = layer.prune_and_regrow(0.1, seed=99)  # on the device
    ref = oracle.topology(300, 400, r, c, v, int(0.1 * r.size), 99)
    assert trials == ref["trials"]
    assert np.array_equal(layer.rows.cpu().numpy(), ref["rows"])
    assert np.array_equal(layer.vals.detach().cpu().numpy().view(np.uint32), ref["vals"].view(np.uint32))
    cv = oracle.build_coo(300, 400, ref["rows"], ref["cols"])
    for k in ("col_perm", "col_rows", "col_cols", "col_offsets"):
        assert np.array_equal(getattr(layer, k).cpu().numpy(), cv[k]), k
    assert layer.vals.device == DEV and layer.col_perm.device == DEV
    X, Y, out = _run(layer, (32,), 700)
    check_close(from_device(Y.detach()), out["Y"], layer.nnz / 300, "regrown Y")
    check_close(layer.vals.grad.cpu().numpy(), out["dW"], 32, "regrown dW")


def test_layer_sgd_reduces_loss_and_save_load_is_exact(tmp_path):
    say("SnackLinear SGD on a fixed regression, save/load")
    torch.manual_seed(0)
    layer = SnackLinear(128, 64, sparsity=0.9, seed=14).to(DEV)
    teacher = SnackLinear(128, 64, sparsity=0.9, seed=14).to(DEV)  # same support, other values below
    with torch.no_grad():
        teacher.vals.mul_(-1.0)
    X = torch.randn(256, 128, device=DEV)
    target = teacher(X).detach()
    opt = torch.optim.SGD(layer.parameters(), lr=0.05)
    losses = []
    for _ in range(30):
        opt.zero_grad()
        loss = ((layer(X) - target) ** 2).sum(dim=1).mean()
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    assert losses[-1] < 0.2 * losses[0], losses
    layer.save_npz(tmp_path / "l.npz")
    back = SnackLinear.load_npz(tmp_path / "l.npz", device=DEV)
    assert torch.equal(back(X), layer(X))


@pytest.mark.parametrize("lead", [(16,), (5,), (64,)], ids=["B16", "B5", "B64"])
def test_column_order_layer_matches_row_order_layer(lead):
    """value_order="col" gives the same outputs and, permuted by col_perm, the same value gradients;
    a few SGD steps and a device prune-and-regrow keep both layers equal bit for bit."""
    say(f"SnackLinear column-order values lead={lead}")
    row = SnackLinear(300, 200, sparsity=0.9, seed=31).to(DEV)
    col = SnackLinear(300, 200, sparsity=0.9, seed=31, value_order="col").to(DEV)
    cp = row.col_perm.long()
    x_in, _ = acts(800, int(np.prod(lead)), 300)
    g_in, _ = acts(801, int(np.prod(lead)), 200)
    X = torch.from_numpy(x_in).to(DEV).reshape(*lead, 300)
    G = torch.from_numpy(g_in).to(DEV).reshape(*lead, 200)
    opt_r = torch.optim.SGD(row.parameters(), lr=0.01)
    opt_c = torch.optim.SGD(col.parameters(), lr=0.01)
    for step in range(3):
        Xr, Xc = X.clone().requires_grad_(True), X.clone().requires_grad_(True)
        Yr, Yc = row(Xr), col(Xc)
        assert torch.equal(Yr, Yc), step
        (Yr * G).sum().backward()
        (Yc * G).sum().backward()
        assert torch.equal(col.vals.grad, row.vals.grad[cp]), step
        assert torch.equal(col.bias.grad, row.bias.grad), step
        check_close(Xc.grad.cpu().numpy(), Xr.grad.cpu().numpy().astype(np.float64), row.nnz / 300, "col dX")
        opt_r.step(); opt_c.step(); opt_r.zero_grad(); opt_c.zero_grad()
    assert torch.equal(col.row_order_vals(), row.vals.detach())
    assert row.prune_and_regrow(0.1, seed=5) == col.prune_and_regrow(0.1, seed=5)
    assert torch.equal(col.rows, row.rows) and torch.equal(col.col_perm, row.col_perm)
    assert torch.equal(col.vals.detach(), row.vals.detach()[row.col_perm.long()])
    assert torch.equal(col.row_to_col[row.col_perm.long()],
                       torch.arange(row.nnz, dtype=torch.int32, device=DEV))
    assert torch.equal(row(X), col(X))
