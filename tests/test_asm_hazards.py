"""The inline-asm DPP moves of the tiled kernels carry their own wait states (CPU only: the kernels'
gfx950 assembly is generated here).

The tiled walks move a broadcast value into a register with an inline-asm v_mov_b32_dpp; the
compiler inserts no wait states for inline asm, so the first move of each chunk carries an
`s_nop 1` (a VALU write of a register followed by a DPP read of it needs two wait states).  This
test compiles snack_coo.hip to device assembly and checks that no v_mov_b32_dpp reads a register
written by a VALU instruction within the two wait states before it."""
import importlib.util
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hip_flags():
    spec = importlib.util.spec_from_file_location("_snack_build", os.path.join(ROOT, "coo_spmm_row_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.HIP_FLAGS


def _hazards(asm_lines):
    """(number of DPP moves checked, list of offending lines)."""
    bad, checked = [], 0
    recent = []  # (VGPR written or None, wait states it accounts for), newest last
    for line in asm_lines:
        t = line.split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        if t.endswith(":"):
            recent = []  # a label: the predecessor is unknown, start over (conservatively clean)
            continue
        if t.startswith("v_mov_b32_dpp") and ("row_newbcast" in t or "quad_perm" in t):
            checked += 1
            src = re.match(r"v_mov_b32_dpp\s+v\d+,\s*(v\d+)", t)
            if src:
                waits = 0
                for dst, w in reversed(recent):
                    if waits >= 2:
                        break
                    if dst == src.group(1):
                        bad.append(t)
                        break
                    waits += w
        nop = re.match(r"s_nop\s+(\d+)", t)
        if nop:
            recent.append((None, int(nop.group(1)) + 1))
        elif t.startswith("v_"):
            m = re.match(r"v_\S+\s+(v\d+)", t)
            recent.append((m.group(1) if m else None, 1))
        else:
            recent.append((None, 1))
        recent = recent[-4:]
    return checked, bad


def test_scan_catches_a_missing_wait_state():
    checked, bad = _hazards(["v_cndmask_b32_e32 v7, 0, v3, vcc",
                             "v_mov_b32_dpp v9, v7 row_newbcast:1 row_mask:0xf bank_mask:0xf"])
    assert checked == 1 and len(bad) == 1
    checked, bad = _hazards(["v_cndmask_b32_e32 v7, 0, v3, vcc", "s_nop 1",
                             "v_mov_b32_dpp v9, v7 row_newbcast:0 row_mask:0xf bank_mask:0xf"])
    assert checked == 1 and not bad


@pytest.mark.timeout(600)
def test_dpp_moves_have_their_wait_states():
    src = os.path.join(ROOT, "coo_spmm_row_amd", "csrc", "snack_coo.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        res = subprocess.run(["hipcc", *_hip_flags(), "--cuda-device-only", "-S", src, "-o", out],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        lines = open(out).read().splitlines()
    checked, bad = _hazards(lines)
    assert checked > 1000  # the tiled kernels' value moves are there
    assert not bad, bad[:5]
