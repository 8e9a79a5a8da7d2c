"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with an
independent fact: the worked example of the SNACK paper (Appendix B, Table 7),
dense brute force on tiny layers, scipy.sparse products, finite differences,
the adjoint identity, special cases, the published SplitMix64 outputs, numpy's
own sort for the builder and the prune order, and the expected trial count of
Algorithm 2 (Section 3.3 / Appendix F).  The mutant tests plant mistakes in a
copy of the oracle source and check that some pin fails for each.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _dense(layer):
    W = np.zeros((layer["out_features"], layer["in_features"]), np.float64)
    W[layer["rows"], layer["cols"]] = layer["vals"].astype(np.float64)
    return W


def _close(a, b, rel=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rel * scale, f"{what}: max abs err {err:g} > {rel * scale:g}"


# ---------------------------------------------------------------- Table 7
def pin_table7():
    g = json.load(open(os.path.join(GOLDEN, "table7.json")))
    dense = np.array(g["dense"], np.float64)
    coo = g["coo"]
    order = [2, 0, 1]  # feed the entries out of order
    rows = np.array(coo["row"])[order]
    cols = np.array(coo["col"])[order]
    vals = np.array(coo["data"], np.float32)[order]
    out = oracle.build_coo(3, 3, rows, cols, vals)
    assert out["rows"].tolist() == coo["row"]
    assert out["cols"].tolist() == g["csr"]["indices"]
    assert out["vals"].tolist() == g["csr"]["data"]
    assert out["row_offsets"].tolist() == g["csr"]["indptr"]
    assert out["vals"][out["col_perm"]].tolist() == g["csc"]["data"]
    assert out["col_rows"].tolist() == g["csc"]["indices"]
    assert out["col_offsets"].tolist() == g["csc"]["indptr"]
    eye = np.eye(3)
    # X = I: Y = X W^T = W^T, so Y[b][o] = A[o][b]
    Y = oracle.fwd(3, 3, out["rows"], out["cols"], out["vals"], eye)
    assert np.array_equal(Y, dense.T)
    # dY = I: dX = dY W = W
    dX = oracle.bwd_input(3, 3, out["rows"], out["cols"], out["vals"], eye)
    assert np.array_equal(dX, dense)
    # dW on the support of A with X = dY = I: (dY^T X)[i,j] = [i == j], zero off the diagonal
    dW = oracle.grad_weight(3, 3, out["rows"], out["cols"], eye, eye)
    assert np.array_equal(dW, np.zeros(3))
    # a single batch row picks out products: X = e_j, dY = e_i  ->  dW[k] = [row_k == i][col_k == j]
    for k in range(3):
        i, j = int(out["rows"][k]), int(out["cols"][k])
        dW = oracle.grad_weight(3, 3, out["rows"], out["cols"], eye[[j]], eye[[i]])
        assert dW.tolist() == [1.0 if kk == k else 0.0 for kk in range(3)]


# ---------------------------------------------------------------- brute force
SMALL_SHAPES = [
    (7, "uniform", 9, 13, 40, 3),
    (8, "one_row", 12, 16, 10, 4),
    (9, "one_col", 16, 11, 9, 2),
    (10, "diag", 10, 10, 10, 5),
    (11, "empty_rows", 24, 20, 60, 6),
    (12, "uniform", 64, 48, 300, 7),
    (13, "uniform", 5, 64, 1, 1),
    (14, "uniform", 33, 1, 20, 3),
]


def pin_bruteforce():
    for seed, shape, O, I, nnz, B in SMALL_SHAPES:
        L = synth.random_small_layer(seed, O, I, nnz, shape)
        W = _dense(L)
        X = synth.make_acts(seed + 100, B, I).astype(np.float64)
        dY = synth.make_acts(seed + 200, B, O).astype(np.float64)
        b = L["bias"].astype(np.float64)
        r, c, v = L["rows"], L["cols"], L["vals"]
        _close(oracle.fwd(O, I, r, c, v, X, L["bias"]), X @ W.T + b, what=f"fwd {shape}")
        _close(oracle.bwd_input(O, I, r, c, v, dY), dY @ W, what=f"dX {shape}")
        _close(oracle.grad_weight(O, I, r, c, X, dY), (dY.T @ X)[r, c], what=f"dW {shape}")
        _close(oracle.grad_bias(dY), dY.sum(axis=0), what=f"db {shape}")


# ---------------------------------------------------------------- scipy.sparse
def pin_scipy(layer_name="tiny", B=4):
    import scipy.sparse as sp
    spec = synth.LAYERS[layer_name]
    L = synth.make_layer(spec)
    O, I = L["out_features"], L["in_features"]
    W = sp.coo_matrix((L["vals"].astype(np.float64), (L["rows"], L["cols"])), shape=(O, I)).tocsr()
    X = synth.make_acts(7, B, I).astype(np.float64)
    dY = synth.make_acts(8, B, O).astype(np.float64)
    Y = oracle.fwd(O, I, L["rows"], L["cols"], L["vals"], X, L["bias"], nthreads=4)
    _close(Y, (W @ X.T).T + L["bias"].astype(np.float64), rel=1e-11, what="fwd vs scipy")
    dX = oracle.bwd_input(O, I, L["rows"], L["cols"], L["vals"], dY, nthreads=4)
    _close(dX, (W.T @ dY.T).T, rel=1e-11, what="dX vs scipy")


# ---------------------------------------------------------------- finite differences
def pin_finite_differences(seed=21, O=40, I=30, nnz=200, B=3):
    """L(vals, X) = <dY, fwd(vals, X)> is linear in vals and in X, so a central
    difference with step 1 equals dW[k] and dX[b,i] up to fp64 rounding."""
    L = synth.random_small_layer(seed, O, I, nnz, "uniform")
    r, c, v = L["rows"], L["cols"], L["vals"].astype(np.float64)
    X = synth.make_acts(seed + 1, B, I).astype(np.float64)
    dY = synth.make_acts(seed + 2, B, O).astype(np.float64)

    def loss(vv, XX):
        return float(np.sum(dY * oracle.fwd(O, I, r, c, vv, XX, None)))

    dW = oracle.grad_weight(O, I, r, c, X, dY)
    dX = oracle.bwd_input(O, I, r, c, v, dY)
    rng = np.random.Generator(np.random.PCG64(seed))
    for k in rng.choice(nnz, size=min(64, nnz), replace=False):
        e = np.zeros(nnz)
        e[k] = 1.0
        fd = (loss(v + e, X) - loss(v - e, X)) / 2.0
        assert abs(fd - dW[k]) <= 1e-10 * max(1.0, abs(dW[k])), ("dW fd", k, fd, dW[k])
    for _ in range(64):
        bi, ii = int(rng.integers(B)), int(rng.integers(I))
        E = np.zeros((B, I))
        E[bi, ii] = 1.0
        fd = (loss(v, X + E) - loss(v, X - E)) / 2.0
        assert abs(fd - dX[bi, ii]) <= 1e-10 * max(1.0, abs(dX[bi, ii])), ("dX fd", bi, ii)


# ---------------------------------------------------------------- adjoint identity
def pin_adjoint(seed=31, O=200, I=150, nnz=3000, B=5):
    """<dY, Y - 1 b^T> = <dX, X> = <dW, vals> (all equal sum_k v_k sum_b dY[b,r_k] X[b,c_k])."""
    L = synth.random_small_layer(seed, O, I, nnz, "uniform")
    r, c, v = L["rows"], L["cols"], L["vals"]
    X = synth.make_acts(seed + 1, B, I)
    dY = synth.make_acts(seed + 2, B, O)
    Y = oracle.fwd(O, I, r, c, v, X, L["bias"])
    dX = oracle.bwd_input(O, I, r, c, v, dY)
    dW = oracle.grad_weight(O, I, r, c, X, dY)
    a = float(np.sum(dY * (Y - L["bias"].astype(np.float64))))
    bb = float(np.sum(dX * X))
    cc = float(np.dot(dW, v.astype(np.float64)))
    scale = float(np.sum(np.abs(dY) @ np.abs(_dense(L)) * np.abs(X))) + 1.0
    assert abs(a - bb) <= 1e-12 * scale and abs(a - cc) <= 1e-12 * scale, (a, bb, cc)


# ---------------------------------------------------------------- special cases
def pin_special_cases():
    L = synth.random_small_layer(41, 30, 20, 120, "empty_rows")
    O, I = 30, 20
    r, c, v, b = L["rows"], L["cols"], L["vals"], L["bias"]
    # X = 0 -> Y = bias exactly; dY = 0 -> dX = 0; X = 0 -> dW = 0
    Y0 = oracle.fwd(O, I, r, c, v, np.zeros((3, I)), b)
    assert np.array_equal(Y0, np.tile(b.astype(np.float64), (3, 1)))
    assert not np.any(oracle.bwd_input(O, I, r, c, v, np.zeros((3, O))))
    assert not np.any(oracle.grad_weight(O, I, r, c, np.zeros((3, I)), np.ones((3, O))))
    # rows without entries output the bias exactly, for any X
    X = synth.make_acts(42, 3, I)
    Y = oracle.fwd(O, I, r, c, v, X, b)
    empty = np.setdiff1d(np.arange(O), r)
    assert empty.size > 0
    assert np.array_equal(Y[:, empty], np.tile(b[empty].astype(np.float64), (3, 1)))
    # single stored entry (r0, c0, w): Y[:, r0] = w X[:, c0] + b[r0]; one dW entry
    r0, c0, w = 4, 7, np.float32(1.75)
    X = synth.make_acts(43, 5, I).astype(np.float64)
    dY = synth.make_acts(44, 5, O).astype(np.float64)
    Y = oracle.fwd(O, I, [r0], [c0], [w], X, b)
    assert np.array_equal(Y[:, r0], 1.75 * X[:, c0] + np.float64(b[r0]))
    others = np.arange(O) != r0
    assert np.array_equal(Y[:, others], np.tile(b[others].astype(np.float64), (5, 1)))
    dW = oracle.grad_weight(O, I, [r0], [c0], X, dY)
    assert dW.shape == (1,) and abs(dW[0] - float(dY[:, r0] @ X[:, c0])) <= 1e-13 * 10
    # diagonal W with I = O: Y = X diag(v) + b, dX = dY diag(v), dW_k = sum_b dY[b,k] X[b,k]
    n = 16
    v = synth.make_acts(45, 1, n)[0]
    X = synth.make_acts(46, 4, n).astype(np.float64)
    dY = synth.make_acts(47, 4, n).astype(np.float64)
    idx = np.arange(n)
    assert np.array_equal(oracle.fwd(n, n, idx, idx, v, X, None), X * v.astype(np.float64))
    assert np.array_equal(oracle.bwd_input(n, n, idx, idx, v, dY), dY * v.astype(np.float64))
    _close(oracle.grad_weight(n, n, idx, idx, X, dY), np.sum(dY * X, axis=0), rel=1e-14)
    # linearity in X
    L = synth.random_small_layer(48, 25, 35, 200, "uniform")
    X1 = synth.make_acts(49, 2, 35).astype(np.float64)
    X2 = synth.make_acts(50, 2, 35).astype(np.float64)
    f = lambda XX: oracle.fwd(25, 35, L["rows"], L["cols"], L["vals"], XX, None)
    _close(f(2.0 * X1 - 3.0 * X2), 2.0 * f(X1) - 3.0 * f(X2), rel=1e-13, what="linearity")


def pin_thread_count_invariance():
    L = synth.random_small_layer(51, 300, 200, 6000, "uniform")
    X = synth.make_acts(52, 9, 200)
    dY = synth.make_acts(53, 9, 300)
    args = (300, 200, L["rows"], L["cols"])
    for nt in (2, 8):
        assert np.array_equal(oracle.fwd(*args, L["vals"], X, L["bias"], nthreads=1),
                              oracle.fwd(*args, L["vals"], X, L["bias"], nthreads=nt))
        assert np.array_equal(oracle.bwd_input(*args, L["vals"], dY, nthreads=1),
                              oracle.bwd_input(*args, L["vals"], dY, nthreads=nt))
        assert np.array_equal(oracle.grad_weight(*args, X, dY, nthreads=1),
                              oracle.grad_weight(*args, X, dY, nthreads=nt))


# ---------------------------------------------------------------- builder vs numpy sort
def pin_builder_numpy(seed=61, O=300, I=170, nnz=4000):
    L = synth.random_small_layer(seed, O, I, nnz, "uniform")
    rng = np.random.Generator(np.random.PCG64(seed))
    shuffle = rng.permutation(nnz)
    r, c, v = L["rows"][shuffle], L["cols"][shuffle], L["vals"][shuffle]
    out = oracle.build_coo(O, I, r, c, v)
    order = np.lexsort((c, r))
    assert np.array_equal(out["perm"], order)
    assert np.array_equal(out["rows"], r[order]) and np.array_equal(out["cols"], c[order])
    assert np.array_equal(out["vals"].view(np.uint32), v[order].view(np.uint32))
    assert np.array_equal(out["row_offsets"], np.searchsorted(r[order], np.arange(O + 1), side="left"))
    corder = np.lexsort((out["rows"], out["cols"]))
    assert np.array_equal(out["col_perm"], corder)
    assert np.array_equal(out["col_rows"], out["rows"][corder])
    assert np.array_equal(out["col_cols"], out["cols"][corder])
    assert np.array_equal(out["col_offsets"], np.searchsorted(out["cols"][corder], np.arange(I + 1)))


def pin_builder_errors():
    def kind(*a):
        try:
            oracle.build_coo(*a)
        except oracle.OracleError as e:
            return e.kind
        return "ok"
    assert kind(4, 4, [0, 1, 0], [1, 2, 1], [1, 2, 3]) == "duplicate"
    assert kind(4, 4, [0, 4], [0, 0], [1, 2]) == "index"
    assert kind(4, 4, [0, -1], [0, 0], [1, 2]) == "index"
    assert kind(4, 4, [0, 1], [0, 4], [1, 2]) == "index"
    assert kind(2, 2, [0, 0, 1, 1, 0], [0, 1, 0, 1, 0], [1] * 5) == "shape"
    assert kind(4, 4, [], [], []) == "ok"
    out = oracle.build_coo(4, 4, [], [], [])
    assert out["row_offsets"].tolist() == [0] * 5 and out["col_offsets"].tolist() == [0] * 5


# ---------------------------------------------------------------- topology update
def pin_splitmix64():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))
    got = ["%016x" % int(x) for x in oracle.splitmix64(g["seed"], len(g["outputs_hex"]))]
    assert got == g["outputs_hex"], got
    # getrand(2^j) keeps the top j bits of each output (multiply-high range reduction)
    ref = [int(h, 16) for h in g["outputs_hex"]]
    for j in (1, 7, 20, 33):
        assert oracle.getrand(g["seed"], 1 << j, len(ref)).tolist() == [u >> (64 - j) for u in ref]


def _topology_case(seed=71, O=60, I=45, nnz=900, frac=0.1):
    L = synth.random_small_layer(seed, O, I, nnz, "uniform")
    # a block of equal magnitudes (both signs) that straddles the prune cut, so the
    # tie-break by position decides which of them go
    v = L["vals"].copy()
    v[::18] = np.float32(0.01)
    v[9::18] = np.float32(-0.01)
    p = int(math.floor(frac * nnz))
    return L, v, p


def pin_topology_invariants():
    for seed in (71, 72, 73):
        L, v, p = _topology_case(seed)
        O, I, nnz = L["out_features"], L["in_features"], L["nnz"]
        out = oracle.topology(O, I, L["rows"], L["cols"], v, p, seed=1234 + seed)
        k = np.arange(nnz)
        prune_order = np.lexsort((k, np.abs(v)))[:p]
        assert np.array_equal(np.sort(prune_order), out["pruned"]), "pruned set"
        keep = np.ones(nnz, bool)
        keep[prune_order] = False
        key_new = out["rows"].astype(np.int64) * I + out["cols"]
        assert out["rows"].size == nnz
        assert np.all(np.diff(key_new) > 0), "sorted and unique"
        assert np.array_equal(out["row_offsets"], np.searchsorted(out["rows"], np.arange(O + 1)))
        key_old = L["rows"].astype(np.int64) * I + L["cols"]
        surv = dict(zip(key_old[keep].tolist(), v[keep].view(np.uint32).tolist()))
        new_map = dict(zip(key_new.tolist(), out["vals"].view(np.uint32).tolist()))
        for kk, bits in surv.items():
            assert new_map.get(kk) == bits, "survivor kept with its value"
        grown = [kk for kk in key_new.tolist() if kk not in surv]
        assert len(grown) == p
        assert all(new_map[kk] == 0 for kk in grown), "regrown value is +0.0"
        assert out["trials"] >= p


def pin_topology_trials_expectation():
    """Algorithm 2 draws until p fresh pairs are added; with s live positions out of
    N, step i succeeds with probability (N - s - i)/N, so trials is a sum of
    geometric variables with mean sum N/(N-s-i) (Section 3.3 / Appendix F)."""
    O, I, nnz = 40, 30, 1000   # dense enough that rejections are frequent
    L = synth.random_small_layer(81, O, I, nnz, "uniform")
    N = O * I
    p = 500
    s = nnz - p
    succ = (N - s - np.arange(p)) / N
    mean = float(np.sum(1.0 / succ))
    var = float(np.sum((1.0 - succ) / succ ** 2))
    n_runs = 40
    tot = 0
    for t in range(n_runs):
        out = oracle.topology(O, I, L["rows"], L["cols"], L["vals"], p, seed=5000 + t)
        tot += out["trials"]
    avg = tot / n_runs
    assert abs(avg - mean) <= 5.0 * math.sqrt(var / n_runs), (avg, mean, math.sqrt(var / n_runs))


def pin_topology_uniformity():
    """Regrown positions are uniform over the free cells: chi-square on row and column counts.
    Counted are regrown cells outside the old support, which are uniform over the cells
    free before the update, so each row's (column's) expected share is its free-cell share."""
    O, I, nnz = 50, 70, 350
    L = synth.random_small_layer(91, O, I, nnz, "uniform")
    old = np.sort(L["rows"].astype(np.int64) * I + L["cols"])
    free = np.ones(O * I, bool)
    free[old] = False
    free_rows = free.reshape(O, I).sum(axis=1).astype(np.float64)
    free_cols = free.reshape(O, I).sum(axis=0).astype(np.float64)
    rows_c = np.zeros(O)
    cols_c = np.zeros(I)
    for t in range(60):
        out = oracle.topology(O, I, L["rows"], L["cols"], L["vals"], nnz // 2, seed=9000 + t)
        new = np.setdiff1d(out["rows"].astype(np.int64) * I + out["cols"], old)
        rows_c += np.bincount(new // I, minlength=O)
        cols_c += np.bincount(new % I, minlength=I)
    total = rows_c.sum()
    for counts, share in ((rows_c, free_rows), (cols_c, free_cols)):
        exp = total * share / share.sum()
        chi2 = float(np.sum((counts - exp) ** 2 / exp))
        dof = counts.size - 1
        assert chi2 < dof + 6.0 * math.sqrt(2 * dof), (chi2, dof)


def _topology_bruteforce(O, I, rows, cols, vals, p, seed):
    """Appendix G's prune step and Algorithm 2's regrowth written out in plain Python: drop the p
    entries of smallest |w| (ties to the lower position in the sorted triple), then draw trials
    from the pinned SplitMix64 stream -- the row from one output, the column from the next,
    each as floor(u*n/2^64) -- and keep a pair only when it is not live; regrown values are +0.0.
    Returns the sorted (row, col, value-bits) triple and the number of trials."""
    nnz = len(rows)
    mags = [abs(float(np.float32(v))) for v in vals]
    order = sorted(range(nnz), key=lambda k: (mags[k], k))
    gone = set(order[:p])
    live = {}
    for k in range(nnz):
        if k not in gone:
            live[(int(rows[k]), int(cols[k]))] = int(np.float32(vals[k]).view(np.uint32))
    need = nnz - len(live)
    u = iter(int(x) for x in oracle.splitmix64(seed, 2 * (50 * need + 1000)))
    trials = 0
    while len(live) < nnz:
        r = (next(u) * O) >> 64
        c = (next(u) * I) >> 64
        trials += 1
        if (r, c) in live:
            continue
        live[(r, c)] = 0
    pos = sorted(live)
    return ([q[0] for q in pos], [q[1] for q in pos], [live[q] for q in pos], trials)


def pin_topology_bruteforce():
    """The oracle's topology update equals the written-out prune-and-regrow exactly: rows, cols,
    value bits and the trial count.  Cases: ties in |w| straddling the cut, a nearly full layer
    (most draws rejected), one row, one column, zeros among the values, and nothing pruned."""
    cases = []
    L, v, p = _topology_case(71)
    cases.append((L["out_features"], L["in_features"], L["rows"], L["cols"], v, p, 4321))
    F = synth.random_small_layer(17, 12, 10, 115, "uniform")   # 115 of 120 cells live
    cases.append((12, 10, F["rows"], F["cols"], F["vals"], 30, 99))
    R = synth.random_small_layer(18, 1, 50, 30, "uniform")
    cases.append((1, 50, R["rows"], R["cols"], R["vals"], 10, 7))
    C = synth.random_small_layer(19, 40, 1, 25, "uniform")
    cases.append((40, 1, C["rows"], C["cols"], C["vals"], 12, 8))
    Z = synth.random_small_layer(20, 20, 20, 150, "uniform")
    vz = Z["vals"].copy()
    vz[::3] = np.float32(0.0)
    vz[1::7] = np.float32(-0.0)
    cases.append((20, 20, Z["rows"], Z["cols"], vz, 60, 31))
    cases.append((20, 20, Z["rows"], Z["cols"], Z["vals"], 0, 32))
    for O, I, rows, cols, vals, p, seed in cases:
        out = oracle.topology(O, I, rows, cols, vals, p, seed=seed)
        r, c, bits, trials = _topology_bruteforce(O, I, rows, cols, vals, p, seed)
        assert out["rows"].tolist() == r and out["cols"].tolist() == c, (O, I, p, "positions")
        assert out["vals"].view(np.uint32).tolist() == bits, (O, I, p, "value bits")
        assert out["trials"] == trials, (O, I, p, out["trials"], trials)


# ---------------------------------------------------------------- uniform initializer
def _init_bruteforce(O, I, nnz, seed):
    """Algorithm 2 written out in Python over the pinned SplitMix64 outputs: each trial takes the
    row from one output and the column from the next (floor(u*n/2^64)), keeps new pairs only."""
    u = iter(int(x) for x in oracle.splitmix64(seed, 200000))
    drawn, trials = set(), 0
    while len(drawn) < nnz:
        r = (next(u) * O) >> 64
        c = (next(u) * I) >> 64
        trials += 1
        drawn.add((r, c))
    pos = sorted(drawn)
    return (np.array([p[0] for p in pos], np.int32), np.array([p[1] for p in pos], np.int32), trials)


def pin_init_uniform_bruteforce():
    for O, I, nnz, seed in ((7, 5, 35, 3), (7, 5, 12, 4), (1, 40, 25, 5), (30, 1, 30, 6), (23, 31, 300, 7)):
        out = oracle.init_uniform(O, I, nnz, seed)
        rows, cols, trials = _init_bruteforce(O, I, nnz, seed)
        assert np.array_equal(out["rows"], rows) and np.array_equal(out["cols"], cols), (O, I, nnz)
        assert out["trials"] == trials, (out["trials"], trials)
        assert np.array_equal(out["row_offsets"], np.searchsorted(rows, np.arange(O + 1)))


def pin_init_uniform_trials_expectation():
    """Appendix F: step i of Algorithm 2 succeeds with probability (mk - i)/mk, so the trial count
    is a sum of geometric variables with mean sum mk/(mk - i) (about -mk ln(eta) at sparsity eta)."""
    O, I, nnz = 40, 30, 900
    N = O * I
    succ = (N - np.arange(nnz)) / N
    mean = float(np.sum(1.0 / succ))
    var = float(np.sum((1.0 - succ) / succ ** 2))
    n_runs = 40
    avg = sum(oracle.init_uniform(O, I, nnz, 300 + t)["trials"] for t in range(n_runs)) / n_runs
    assert abs(avg - mean) <= 5.0 * math.sqrt(var / n_runs), (avg, mean)
    eta = 1.0 - nnz / N
    assert abs(mean / nnz - (-math.log(eta) / (1.0 - eta))) < 0.02 * mean / nnz  # the pages' closed form


def pin_init_uniform_uniformity():
    """Positions are uniform over the matrix: chi-square on row and column counts."""
    O, I, nnz = 50, 70, 700
    rows_c, cols_c = np.zeros(O), np.zeros(I)
    for t in range(40):
        out = oracle.init_uniform(O, I, nnz, 700 + t)
        rows_c += np.bincount(out["rows"], minlength=O)
        cols_c += np.bincount(out["cols"], minlength=I)
    for counts in (rows_c, cols_c):
        exp = counts.sum() / counts.size
        chi2 = float(np.sum((counts - exp) ** 2 / exp))
        dof = counts.size - 1
        assert chi2 < dof + 6.0 * math.sqrt(2 * dof), (chi2, dof)


ALL_PINS = [
    pin_table7, pin_bruteforce, pin_scipy, pin_finite_differences, pin_adjoint,
    pin_special_cases, pin_thread_count_invariance, pin_builder_numpy, pin_builder_errors,
    pin_splitmix64, pin_topology_invariants, pin_topology_trials_expectation,
    pin_topology_uniformity, pin_topology_bruteforce, pin_init_uniform_bruteforce, pin_init_uniform_trials_expectation,
    pin_init_uniform_uniformity,
]
