"""Re-runs the gfx950 measurements that the tiled kernels' layout rests on (tests/probes, built by
__graft_entry__.build()) and checks the relations the design uses (needs a GPU):

* four 16-lane slots each reading a 256-byte row with ds_read_b128 keep the LDS at full rate when
  their 16-byte chunk positions differ only in the two low bits (chunk j at j ^ (row & 3)), and
  lose rate with the swizzle over all four bits or over bits 2-3;
* staging writes of consecutive rows by consecutive lanes conflict unswizzled and not with the
  low-two-bit swizzle;
* a plain v_fmac_f32 issues faster than its DPP form, which is why a step moves the broadcast value
  into a register once and then uses plain FMAs."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import say  # noqa: E402

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libgfx950_probes.so")


@pytest.fixture(scope="module")
def probes():
    torch.cuda.init()  # one HIP runtime: torch's, loaded first
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built: run __graft_entry__.build()")
    return ctypes.CDLL(LIB)


def _rate(fn, arg):
    r = ctypes.c_double(0.0)
    assert fn(arg, ctypes.byref(r)) == 0
    return r.value


def test_lds_row_swizzle(probes):
    say("LDS probes")
    read = {m: _rate(probes.probe_lds_read, ctypes.c_uint(m)) for m in (0, 3, 12, 15)}
    write = {m: _rate(probes.probe_lds_write, ctypes.c_uint(m)) for m in (0, 3, 15)}
    print("ds_read_b128, 4 slots x 256-byte rows, chunk j at j ^ (row & mask), B/clk/CU:",
          {m: round(v, 1) for m, v in read.items()})
    print("ds_write_b128 staging of consecutive rows, B/clk/CU:", {m: round(v, 1) for m, v in write.items()})
    assert read[3] > 1.2 * read[15] and read[3] > 1.2 * read[12]
    assert write[3] > 2.0 * write[0]


def test_valu_issue_rates(probes):
    say("VALU probes")
    names = ["v_fmac_f32", "v_fmac_f32 (DPP)", "v_mov_b32 (DPP)", "v_xor_b32 (DPP)"]
    rates = [_rate(probes.probe_valu_rate, ctypes.c_int(m)) for m in range(len(names))]
    print("wave-instructions per clock per CU:", {n: round(r, 3) for n, r in zip(names, rates)})
    assert rates[0] > 1.2 * rates[1]
    assert rates[2] > 0.5 and rates[3] > 0.5
