"""snack_coo_fwd_noalloc (workspace in the library's static device scratch) gives the results of
snack_coo_fwd, on two calls in a row, the second with a smaller input (needs a GPU)."""
import pytest

import synth
from gpu_util import device_layer, named_layer, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import coo_spmm_row_amd as snk  # noqa: E402

DEV = torch.device("cuda:0")


def _pair(W, X, bias, O):
    """(snack_coo_fwd, snack_coo_fwd_noalloc) outputs for the same call."""
    B = X.shape[0]
    want = snk.snack_coo_fwd(W, X, bias)
    got = torch.full((B, O), float("nan"), dtype=X.dtype, device=DEV)
    snk.snack_coo_fwd_noalloc(W, X, got, bias)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("bf16", [False, True])
def test_noalloc_forward_matches_forward_twice(bf16):
    """First the 10k x 10k 95 % layer at batch 64 (tiled: about 42 MB of block partials in the
    scratch), then a smaller layer at batch 8: bit-equal to snack_coo_fwd both times."""
    spec, L = named_layer("target95")
    O, I = L["out_features"], L["in_features"]
    built, W = device_layer(L, DEV)
    dt = torch.bfloat16 if bf16 else torch.float32
    X = to_device(synth.make_acts(11, 64, I), DEV).to(dt)
    bias = torch.from_numpy(L["bias"]).to(DEV)
    need = snk.snack_coo_workspace_bytes(snk.OP_FWD, W, 64, snk.SNACK_BF16 if bf16 else snk.SNACK_F32)
    say(f"noalloc 1: target95 B=64 bf16={bf16} workspace {need} bytes")
    assert 0 < need <= snk.NOALLOC_SCRATCH_BYTES
    got, want = _pair(W, X, bias, O)
    assert torch.equal(got, want)

    L2 = synth.random_small_layer(173, 500, 700, 20000, "empty_rows")
    built2, W2 = device_layer(L2, DEV)
    X2 = to_device(synth.make_acts(12, 8, 700), DEV).to(dt)
    bias2 = torch.from_numpy(L2["bias"]).to(DEV)
    say(f"noalloc 2: 500 x 700 B=8 bf16={bf16}")
    got2, want2 = _pair(W2, X2, bias2, 500)
    assert torch.equal(got2, want2)


def test_noalloc_forward_refuses_oversized_call():
    """A call needing more workspace than the scratch holds fails with SNACK_ERR_WORKSPACE and
    leaves the output untouched."""
    spec, L = named_layer("target95")
    built, W = device_layer(L, DEV)
    B = 4096
    need = snk.snack_coo_workspace_bytes(snk.OP_FWD, W, B, snk.SNACK_F32)
    say(f"noalloc oversized: B={B} workspace {need} bytes")
    assert need > snk.NOALLOC_SCRATCH_BYTES
    X = torch.zeros(B, L["in_features"], device=DEV)
    Y = torch.full((B, L["out_features"]), 3.0, device=DEV)
    with pytest.raises(RuntimeError, match="static scratch"):
        snk.snack_coo_fwd_noalloc(W, X, Y)
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all())
