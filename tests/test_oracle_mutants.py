"""Plant plausible mistakes in a copy of the oracle source (CPU only) and check
that at least one pin catches each of them.  Each mutant is compiled with gcc
into a temporary library and exercised in a child process, so a mutant that
crashes (for example by writing out of bounds) also counts as caught."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "snack_oracle.c")

# (name, text to replace, replacement)
MUTANTS = [
    ("fwd_transposed_operand", "y[rows[k]] += vals[k] * x[cols[k]]", "y[rows[k]] += vals[k] * x[rows[k] % I]"),
    ("fwd_sign", "y[rows[k]] += vals[k] * x[cols[k]]", "y[rows[k]] -= vals[k] * x[cols[k]]"),
    ("fwd_no_bias", "if (bias) for (int64_t i = 0; i < O; ++i) y[i] += bias[i];", ""),
    ("fwd_bias_twice", "y[i] += bias[i];", "y[i] += 2.0 * bias[i];"),
    ("fwd_skip_last_entry", "for (int64_t k = 0; k < nnz; ++k) y[rows[k]]", "for (int64_t k = 0; k + 1 < nnz; ++k) y[rows[k]]"),
    ("dx_wrong_index", "dx[cols[k]] += vals[k] * dy[rows[k]]", "dx[cols[k]] += vals[k] * dy[cols[k] % O]"),
    ("dx_no_transpose", "dx[cols[k]] += vals[k] * dy[rows[k]]", "dx[rows[k] % I] += vals[k] * dy[cols[k] % O]"),
    ("dw_wrong_operand", "s += dY[t * O + rows[k]] * X[t * I + cols[k]]", "s += dY[t * O + rows[k]] * X[t * I + rows[k] % I]"),
    ("dw_dropped_batch_term", "for (int64_t t = 0; t < B; ++t) s += dY[t * O + rows[k]]", "for (int64_t t = 1; t < B; ++t) s += dY[t * O + rows[k]]"),
    ("dw_accumulates", "dW[k] = s;", "dW[k] += s;"),
    ("db_dropped_term", "for (int64_t t = 0; t < B; ++t) s += dY[t * O + i];", "for (int64_t t = 0; t + 1 < B; ++t) s += dY[t * O + i];"),
    ("build_offsets_shift", "row_offsets_out[rows[e[k].idx] + 1] += 1", "row_offsets_out[rows[e[k].idx]] += 1"),
    ("build_no_dup_check", "if (e[k].key == e[k - 1].key) { free(e); return OR_DUP; }", ""),
    ("build_colview_rowmajor", "t[k].key = (int64_t)cols[src] * O + rows[src];", "t[k].key = (int64_t)rows[src] * I + cols[src];"),
    ("build_key_colmajor", "e[k].key = (int64_t)rows[k] * I + cols[k];", "e[k].key = (int64_t)cols[k] * O + rows[k];"),
    ("build_no_range_check", "if (rows[k] < 0 || rows[k] >= O || cols[k] < 0 || cols[k] >= I) return OR_INDEX;\n    }", "}"),
    ("splitmix_constant", "0xBF58476D1CE4E5B9ULL", "0xBF58476D1CE4E5B8ULL"),
    ("getrand_modulo", "return (int64_t)(p >> 64);", "return (int64_t)(splitmix64_next(state) % (uint64_t)n) + 0 * (int64_t)(p >> 64);"),
    ("prune_tiebreak_reversed", "return (x->k > y->k) - (x->k < y->k);\n}\n\n/* Input", "return (x->k < y->k) - (x->k > y->k);\n}\n\n/* Input"),
    ("prune_by_signed_value", "m[k].mag = fabsf(vals[k]);", "m[k].mag = vals[k];"),
    ("regrow_value_not_zero", "v2[n2] = 0.0f;", "v2[n2] = 1.0f;"),
    ("regrow_no_set_insert", "live[i * I + j] = 1;\n        r2[n2]", "r2[n2]"),
    ("regrow_trials_miscount", "++trials;\n        if (live[i * I + j]) continue;", "if (live[i * I + j]) continue;\n        ++trials;"),
    ("regrow_swapped_ranges", "int64_t i = getrand(&state, O);\n        int64_t j = getrand(&state, I);",
     "int64_t i = getrand(&state, I) % O;\n        int64_t j = getrand(&state, O) % I;"),
    ("regrow_column_first", "int64_t i = getrand(&state, O);\n        int64_t j = getrand(&state, I);",
     "int64_t j = getrand(&state, I);\n        int64_t i = getrand(&state, O);"),
    ("init_column_first", "const int64_t row = getrand(&state, O);   /* row first, then column */\n        const int64_t col = getrand(&state, I);",
     "const int64_t col = getrand(&state, I);\n        const int64_t row = getrand(&state, O);"),
    ("init_no_rejection", "if (seen[row * I + col]) continue;         /* drawn before: reject */", ""),
    ("init_trials_counts_accepted_only", "trials += 1;\n        if (seen[row * I + col]) continue;",
     "if (seen[row * I + col]) continue;\n        trials += 1;"),
    ("init_no_set_insert", "seen[row * I + col] = 1;\n        r[n]", "r[n]"),
]

RUNNER = r"""
import ctypes, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
oracle._lib = oracle.configure(ctypes.CDLL({lib!r}))
import pins
failed = []
for pin in pins.ALL_PINS:
    try:
        pin()
    except Exception as e:  # noqa: BLE001
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mutated = src.replace(old, new)
    csrc = tmp_path / "mut.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(csrc), "-lm"],
                   check=True, capture_output=True)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(lib))
    try:
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        return  # a mutant that never finishes is caught as well
    if res.returncode != 0:
        return  # crashed: caught
    line = [ln for ln in res.stdout.splitlines() if ln.startswith("FAILED_PINS")]
    assert line, res.stdout + res.stderr
    failed = line[0].split(" ", 1)[1] if " " in line[0] else ""
    assert failed.strip(), f"mutant {name} passed every pin"
