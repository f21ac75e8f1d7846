"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Each pin is a function ``pin_*(o)`` taking a loaded :class:`oracle.Oracle` and
raising ``AssertionError`` when the oracle disagrees.  ``test_oracle_pins.py``
runs them on the oracle; ``test_oracle_mutants.py`` runs them on copies of the
oracle with a planted mistake and requires each mistake to trip at least one.

Sources: [P2] V. Dubrov, "DeepSeek mHC: Manifold-Constrained Hyper-Connections"
(slavadubrov.com); [P5] "mHC" study notes on DeepSeek-V4 (t6page.pages.dev).
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    sections, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                sections[cur] = []
            else:
                sections[cur].append(line.split())
    return sections


def _mat(rows):
    return np.array([[float(v) for v in r] for r in rows])


def _close3(got, printed):
    """Agreement with a value printed to 3 decimals."""
    assert np.all(np.abs(np.asarray(got) - np.asarray(printed)) <= 5e-4 + 1e-12), (got, printed)


# --------------------------------------------------------------------------
# Sinkhorn-Knopp: [P2] Sinkhorn-Knopp-projectie (procedure, 3x3 example);
# [P5] eqs. dsv4-mhc-sinkhorn-init, dsv4-mhc-sinkhorn.

def pin_sinkhorn_page_3x3(o):
    """The page's worked 3x3 example: exp, one pass, twenty passes."""
    g = _read_golden("sinkhorn_3x3.txt")
    A = _mat(g["logits"])
    _close3(o.sinkhorn(A, 0), _mat(g["exp"]))
    M1 = o.sinkhorn(A, 1)
    _close3(M1, _mat(g["pass1"]))
    _close3(M1.sum(axis=1), _mat(g["pass1_row_sums"])[0])
    _close3(M1.sum(axis=0), _mat(g["pass1_col_sums"])[0])
    M20 = o.sinkhorn(A, 20)
    _close3(M20, _mat(g["pass20"]))
    _close3(M20.sum(axis=1), _mat(g["pass20_row_sums"])[0])
    _close3(M20.sum(axis=0), _mat(g["pass20_col_sums"])[0])


def _sk_scaling_vectors(L, t_max):
    """Independent formulation: M = diag(u) E diag(v), updating v (column step)
    then u (row step); the iterates equal those of alternating normalisation."""
    E = [[math.exp(v) for v in row] for row in L]
    n = len(E)
    u = [1.0] * n
    v = [1.0] * n
    for _ in range(t_max):
        v = [1.0 / sum(u[i] * E[i][j] for i in range(n)) for j in range(n)]
        u = [1.0 / sum(E[i][j] * v[j] for j in range(n)) for i in range(n)]
    return np.array([[u[i] * E[i][j] * v[j] for j in range(n)] for i in range(n)])


def pin_sinkhorn_scaling_vectors(o):
    """Brute force against the diagonal-scaling form, n = 1..5, several t."""
    rng = np.random.default_rng(11)
    for n in (1, 2, 3, 4, 5):
        for t in (1, 2, 5, 20):
            L = rng.normal(0.0, 1.5, (n, n))
            ref = _sk_scaling_vectors(L.tolist(), t)
            got = o.sinkhorn(L, t)
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-15), (n, t, got, ref)


def pin_sinkhorn_n2_closed_form(o):
    """n = 2: scaling keeps the cross ratio M11 M22 / (M12 M21) = exp(D),
    D = l11 + l22 - l12 - l21, and the only doubly stochastic 2x2 matrices
    are [[a, 1-a], [1-a, a]], so the limit has a = sigmoid(D / 2)."""
    rng = np.random.default_rng(12)
    for _ in range(20):
        L = rng.normal(0.0, 1.0, (2, 2))
        D = L[0, 0] + L[1, 1] - L[0, 1] - L[1, 0]
        a = 1.0 / (1.0 + math.exp(-D / 2.0))
        ref = np.array([[a, 1 - a], [1 - a, a]])
        got = o.sinkhorn(L, 400)                        # the limit
        assert np.allclose(got, ref, rtol=0, atol=1e-13), (D, got, ref)
        if abs(D) <= 1.2:                               # already there after 20 passes
            assert np.allclose(o.sinkhorn(L, 20), ref, rtol=0, atol=1e-13), (D, got, ref)


def pin_sinkhorn_checkpoints(o):
    """Doubly stochastic within tolerance at the workloads' bias scale:
    after the 20th column step the column sums are 1 to 1e-6 and the row sums
    to 1e-3; after the final row step the row sums are 1 to 1e-6 and the
    column sums to 1e-3.  All entries stay positive."""
    rng = np.random.default_rng(13)
    for _ in range(200):
        L = 2.0 * np.eye(4) + rng.normal(0.0, 0.1, (4, 4)) + rng.normal(0.0, 0.08, (4, 4))
        M, tr = o.sinkhorn(L, 20, trace=True)
        rows_c, cols_c = tr[19, 0, 0], tr[19, 0, 1]
        rows_r, cols_r = tr[19, 1, 0], tr[19, 1, 1]
        assert np.max(np.abs(cols_c - 1)) <= 1e-6 and np.max(np.abs(rows_c - 1)) <= 1e-3
        assert np.max(np.abs(rows_r - 1)) <= 1e-6 and np.max(np.abs(cols_r - 1)) <= 1e-3
        assert np.all(M > 0)
        assert np.allclose(M.sum(axis=1), rows_r, rtol=0, atol=1e-14)


def pin_sinkhorn_shift_and_permutation(o):
    """Adding a constant to every logit changes nothing (the first column step
    removes it); permuting rows and columns of the logits permutes the result."""
    rng = np.random.default_rng(14)
    for _ in range(10):
        L = rng.normal(0.0, 1.0, (4, 4))
        base = o.sinkhorn(L, 20)
        assert np.allclose(o.sinkhorn(L + 3.7, 20), base, rtol=1e-12, atol=1e-15)
        p, q = rng.permutation(4), rng.permutation(4)
        assert np.allclose(o.sinkhorn(L[p][:, q], 20), base[p][:, q], rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# Composite map and Amax: [P2] "Het probleem van de samengestelde map" and the
# NumPy demo in "Sinkhorn-Knopp-projectie".

def _stack_from_mats(mats, n):
    L = len(mats)
    H = np.zeros((L, 1, n * n + 2 * n))
    for l, a in enumerate(mats):
        H[l, 0, n:n + n * n] = np.asarray(a).reshape(-1)
    return H


def pin_amax_page_demo(o):
    """The page's seed-0 demo: 1906.8 for HC, 1.0 for mHC (one decimal)."""
    g = _read_golden("amax_demo_seed0.txt")
    printed = {k: float(v) for k, v in g["printed"]}
    rng = np.random.default_rng(0)
    mats = [np.eye(4) + 0.3 * rng.standard_normal((4, 4)) for _ in range(60)]
    hc = o.amax(_stack_from_mats(mats, 4), 4)["amax"][0]
    mhc = o.amax(_stack_from_mats([o.sinkhorn(a, 20) for a in mats], 4), 4)["amax"][0]
    assert round(hc, 1) == printed["hc"], hc
    assert round(mhc, 1) == printed["mhc"], mhc


def pin_amax_hand_product(o):
    """Two hand-multiplied 2x2 maps.  H1 = [[1,-2],[0,1]], H2 = [[1,0],[3,1]]:
    H2 H1 = [[1,-2],[3,-5]] -> abs row sums 3, 8 and abs column sums 4, 7.
    (H1 H2 = [[-5,-2],[3,1]] would give rows 7, 4 and columns 8, 3.)"""
    H1 = [[1.0, -2.0], [0.0, 1.0]]
    H2 = [[1.0, 0.0], [3.0, 1.0]]
    r = o.amax(_stack_from_mats([H1, H2], 2), 2)
    assert np.array_equal(r["composite"][0], np.array([[1.0, -2.0], [3.0, -5.0]]))
    assert r["gain_fwd"][0] == 8.0 and r["gain_bwd"][0] == 7.0 and r["amax"][0] == 8.0
    r1 = o.amax(_stack_from_mats([[[1.0, 2.0], [0.0, -0.5]]], 2), 2)   # rows 3, 0.5; columns 1, 2.5
    assert r1["gain_fwd"][0] == 3.0 and r1["gain_bwd"][0] == 2.5
    r0 = o.amax(np.zeros((0, 1, 8)), 2)
    assert np.array_equal(r0["composite"][0], np.eye(2)) and r0["amax"][0] == 1.0


def pin_amax_closure(o):
    """A product of doubly stochastic maps is doubly stochastic (closure):
    after the final row step every map's row sums are exactly 1 (to rounding),
    so the composite's row sums are 1; column sums stay within the sum of the
    per-layer column errors."""
    rng = np.random.default_rng(15)
    mats = [o.sinkhorn(2.0 * np.eye(4) + rng.normal(0, 0.5, (4, 4)), 20) for _ in range(60)]
    r = o.amax(_stack_from_mats(mats, 4), 4)
    P = r["composite"][0]
    col_err = sum(np.max(np.abs(m.sum(axis=0) - 1)) for m in mats)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert np.max(np.abs(P.sum(axis=0) - 1)) <= col_err + 1e-12
    assert abs(r["gain_fwd"][0] - 1.0) <= 1e-12


# --------------------------------------------------------------------------
# Layer maps: [P5] eqs. dsv4-mhc-rmsnorm, a/b/c-tilde, gate; aggregation and
# mixing: [P2] "Kernmechanismen" Eq. 3, [P5] eq. dsv4-mhc-hc-update.

def _layer_inputs(rng, T, n, d, alpha=(0.01, 0.01, 0.01), bres=2.0):
    m = n * n + 2 * n
    X = rng.normal(0.0, 1.0, (T, n, d)).astype(np.float32)
    phi = rng.normal(0.0, 0.02, (n * d, m)).astype(np.float32)
    bias = rng.normal(0.0, 0.1, m).astype(np.float32)
    bias[n:n + n * n] += (bres * np.eye(n)).reshape(-1).astype(np.float32)
    Y = rng.normal(0.0, 1.0, (T, d)).astype(np.float32)
    return X, phi, bias, np.array(alpha, dtype=np.float32), Y


def pin_gates_closed_form(o):
    """alpha = 0 leaves only the static biases.  sigmoid(ln 3) = 3/4,
    sigmoid(-ln 3) = 1/4, sigmoid(0) = 1/2; the write map doubles them, so a
    zero logit writes with weight 1; zero residual logits give 1/n everywhere."""
    n, d = 4, 8
    X = np.ones((1, n, d), dtype=np.float32)
    phi = np.ones((n * d, n * n + 2 * n), dtype=np.float32)
    l3 = math.log(3.0)
    bias = np.zeros(n * n + 2 * n, dtype=np.float32)
    bias[:n] = [l3, -l3, 0.0, l3]
    bias[n + n * n:] = [0.0, -l3, l3, 0.0]
    r = o.pre(X, phi, bias, (0.0, 0.0, 0.0))
    H = r["H"][0]
    assert np.allclose(H[:n], [0.75, 0.25, 0.5, 0.75], rtol=0, atol=1e-7)
    assert np.allclose(H[n + n * n:], [1.0, 0.5, 1.5, 1.0], rtol=0, atol=1e-7)
    assert np.allclose(H[n:n + n * n], 0.25, rtol=0, atol=1e-15)


def pin_rmsnorm_onehot(o):
    """Constant streams X[t, i, :] = c_i give r = sqrt(sum_i c_i^2 / n + eps)
    over the whole flattened state; a one-hot phi column picking element
    (i0, c0) of vec(X) (stream i0 at [i0 d, (i0+1) d)) gives z = c_i0 / r."""
    n, d, m = 4, 8, 24
    c = np.array([0.5, -1.25, 2.0, 0.125]) * 1e-3       # small: eps = 1e-6 matters
    X = np.broadcast_to(c[None, :, None], (1, n, d)).astype(np.float32).copy()
    eps = 1e-6
    r_ref = math.sqrt(float(np.sum(c.astype(np.float32).astype(np.float64) ** 2)) / n + eps)
    for (i0, c0, j0) in ((0, 0, 0), (2, 5, 7), (3, 7, 23), (1, 3, 12)):
        phi = np.zeros((n * d, m), dtype=np.float32)
        phi[i0 * d + c0, j0] = 1.0
        r = o.pre(X, phi, np.zeros(m, np.float32), (1.0, 1.0, 1.0), eps=eps, extras=True)
        assert abs(r["r"][0] - r_ref) <= 1e-15, (r["r"][0], r_ref)
        z = r["z"][0]
        xi = float(np.float32(c[i0]))
        assert abs(z[j0] - xi / r_ref) <= 1e-12 and np.count_nonzero(z) == 1, (i0, c0, j0, z)


def pin_projection_blocks_and_mat(o):
    """Column blocks pre | res | post take alpha_pre, alpha_res, alpha_post;
    Mat() is row-major with row = output stream: a large logit in column
    n + i*n + j makes entry (i, j) the largest of its row and its column."""
    n, d, m = 4, 4, 24
    rng = np.random.default_rng(16)
    X = rng.normal(0, 1, (1, n, d)).astype(np.float32)
    x = X.reshape(-1).astype(np.float64)
    r = math.sqrt(float(np.mean(x * x)) + 1e-6)
    alpha = (0.5, 2.0, -1.5)
    phi = np.zeros((n * d, m), dtype=np.float32)
    for j in range(m):
        phi[j % (n * d), j] = 1.0               # column j reads element j mod 16 of vec(X)
    bias = rng.normal(0, 0.1, m).astype(np.float32)
    out = o.pre(X, phi, bias, alpha, extras=True)
    for j in range(m):
        a = alpha[0] if j < n else alpha[1] if j < n + n * n else alpha[2]
        expect = a * x[j % (n * d)] / r + float(bias[j])
        assert abs(out["logit"][0][j] - expect) <= 1e-12, (j, out["logit"][0][j], expect)
    for (i, j) in ((1, 2), (3, 0), (0, 3)):
        b = np.zeros(m, np.float32)
        b[n + i * n + j] = 6.0
        Hres = o.pre(X, phi, b, (0.0, 0.0, 0.0))["H"][0][n:n + n * n].reshape(n, n)
        assert np.argmax(Hres[i]) == j and np.argmax(Hres[:, j]) == i, Hres


def _naive_layer(X, Y, phi, bias, alpha, eps, t_max):
    """Independent fp64 formulation: reordered RMSNorm (x . phi) / r with
    numpy's matmul, diagonal-scaling Sinkhorn, einsum aggregation/mixing."""
    T, n, d = X.shape
    m = n * n + 2 * n
    Xd = X.astype(np.float64)
    x = Xd.reshape(T, n * d)
    r = np.sqrt(np.mean(x * x, axis=1) + eps)
    z = (x @ phi.astype(np.float64)) / r[:, None]
    a = np.concatenate([np.full(n, alpha[0]), np.full(n * n, alpha[1]), np.full(n, alpha[2])]).astype(np.float64)
    lg = a[None, :] * z + bias.astype(np.float64)[None, :]
    Hpre = 1.0 / (1.0 + np.exp(-lg[:, :n]))
    Hpost = 2.0 / (1.0 + np.exp(-lg[:, n + n * n:]))
    Hres = np.stack([_sk_scaling_vectors(lg[t, n:n + n * n].reshape(n, n).tolist(), t_max) for t in range(T)])
    h = np.einsum("ti,tid->td", Hpre, Xd)
    H = np.concatenate([Hpre, Hres.reshape(T, n * n), Hpost], axis=1)
    Hf = H.astype(np.float32).astype(np.float64)
    Xo = np.einsum("tij,tjd->tid", Hf[:, n:n + n * n].reshape(T, n, n), Xd) \
        + Hf[:, n + n * n:, None] * Y.astype(np.float64)[:, None, :]
    return h, H, Xo


def pin_bruteforce_tiny_layers(o):
    """Whole layer on tiny shapes against the independent formulation."""
    rng = np.random.default_rng(17)
    for n in (1, 2, 3, 4, 8):
        for d in (1, 3, 8):
            for alpha in ((0.01, 0.01, 0.01), (1.0, 0.7, -0.4)):
                T = 3
                X, phi, bias, al, Y = _layer_inputs(rng, T, n, d, alpha)
                h_ref, H_ref, Xo_ref = _naive_layer(X, Y, phi, bias, al, 1e-6, 20)
                out = o.pre(X, phi, bias, al, eps=1e-6, t_max=20)
                assert np.allclose(out["H"], H_ref, rtol=1e-11, atol=1e-14), (n, d, alpha)
                assert np.allclose(out["h"], h_ref, rtol=1e-11, atol=1e-13), (n, d, alpha)
                Xo = o.post(X, Y, out["H"].astype(np.float32))
                assert np.allclose(Xo, Xo_ref, rtol=1e-11, atol=1e-13), (n, d, alpha)


def pin_alpha0_closed_form(o):
    """alpha = 0 and F = 0: every token gets the same maps, X' = H_res X with
    H_res = SK(exp(b_res)), and h = sum_i sigmoid(b_pre,i) X_i."""
    rng = np.random.default_rng(18)
    n, d, T = 4, 16, 5
    X, phi, bias, _, _ = _layer_inputs(rng, T, n, d)
    Y = np.zeros((T, d), np.float32)
    out = o.pre(X, phi, bias, (0.0, 0.0, 0.0))
    Hres = o.sinkhorn(bias[n:n + n * n].astype(np.float64).reshape(n, n), 20)
    spre = 1.0 / (1.0 + np.exp(-bias[:n].astype(np.float64)))
    for t in range(T):
        assert np.allclose(out["H"][t, n:n + n * n].reshape(n, n), Hres, rtol=1e-14, atol=0)
        assert np.allclose(out["h"][t], spre @ X[t].astype(np.float64), rtol=1e-12, atol=1e-14)
    Xo = o.post(X, Y, out["H"].astype(np.float32))
    Hf = out["H"][0, n:n + n * n].astype(np.float32).astype(np.float64).reshape(n, n)
    for t in range(T):
        assert np.allclose(Xo[t], Hf @ X[t].astype(np.float64), rtol=1e-12, atol=1e-14)


def pin_single_stream_is_residual(o):
    """n = 1: H_res = [1] exactly, and with a zero write logit the layer is the
    standard residual X' = X + F; generally X' = X + 2 sigmoid(l_post) Y."""
    rng = np.random.default_rng(19)
    X, phi, bias, al, Y = _layer_inputs(rng, 4, 1, 8, (0.3, 0.3, 0.3))
    out = o.pre(X, phi, bias, al, extras=True)
    assert np.all(out["H"][:, 1] == 1.0)
    Xo = o.post(X, Y, out["H"].astype(np.float32))
    wpost = out["H"][:, 2].astype(np.float32).astype(np.float64)
    assert np.allclose(Xo[:, 0], X[:, 0].astype(np.float64) + wpost[:, None] * Y, rtol=1e-13, atol=1e-14)
    b0 = np.zeros(3, np.float32)
    out0 = o.pre(X, phi, b0, (0.0, 0.0, 0.0))
    Xo0 = o.post(X, Y, out0["H"].astype(np.float32))
    assert np.allclose(Xo0[:, 0], X[:, 0].astype(np.float64) + Y.astype(np.float64), rtol=1e-14, atol=0)


def pin_equal_streams_and_conservation(o):
    """Rows of H_res sum to 1 after the last row step, so identical streams
    pass through unchanged (F = 0); columns sum to 1 within the column error,
    so the stream sum is conserved up to the write term."""
    rng = np.random.default_rng(20)
    n, d, T = 4, 16, 6
    _, phi, bias, al, Y = _layer_inputs(rng, T, n, d)
    x = rng.normal(0, 1, (T, 1, d)).astype(np.float32)
    Xeq = np.repeat(x, n, axis=1)
    out = o.pre(Xeq, phi, bias, al, extras=True)
    Xo = o.post(Xeq, np.zeros((T, d), np.float32), out["H"].astype(np.float32))
    rowerr = np.abs(out["H"][:, n:n + n * n].astype(np.float32).astype(np.float64).reshape(T, n, n).sum(axis=2) - 1).max()
    xmax = float(np.abs(x).max())
    assert np.allclose(Xo, Xeq.astype(np.float64), rtol=0, atol=rowerr * xmax * 1.0001 + 1e-12)
    X = rng.normal(0, 1, (T, n, d)).astype(np.float32)
    out = o.pre(X, phi, bias, al, extras=True)
    assert np.all(out["sk_err"][:, 2] <= 1e-3)
    Xo = o.post(X, Y, out["H"].astype(np.float32))
    Hf = out["H"].astype(np.float32).astype(np.float64)
    lhs = Xo.sum(axis=1)
    rhs = X.astype(np.float64).sum(axis=1) + Hf[:, n + n * n:].sum(axis=1)[:, None] * Y
    colerr = np.abs(Hf[:, n:n + n * n].reshape(T, n, n).sum(axis=1) - 1).max(axis=1)
    bound = colerr[:, None] * np.abs(X.astype(np.float64)).sum(axis=1) + 1e-12
    assert np.all(np.abs(lhs - rhs) <= bound)


def pin_streams_really_mix(o):
    """A residual map pinned near a 4-cycle permutation P (logits 30 P) must
    route input stream pi(i) to output stream i, where P[i, pi(i)] = 1."""
    n, d, T = 4, 8, 2
    rng = np.random.default_rng(21)
    pi = [1, 2, 3, 0]
    P = np.zeros((n, n))
    for i in range(n):
        P[i, pi[i]] = 1.0
    bias = np.zeros(n * n + 2 * n, np.float32)
    bias[n:n + n * n] = (30.0 * P).reshape(-1)
    X = rng.normal(0, 1, (T, n, d)).astype(np.float32)
    phi = np.zeros((n * d, n * n + 2 * n), np.float32)
    out = o.pre(X, phi, bias, (0.0, 0.0, 0.0))
    Xo = o.post(X, np.zeros((T, d), np.float32), out["H"].astype(np.float32))
    for i in range(n):
        assert np.allclose(Xo[:, i], X[:, pi[i]].astype(np.float64), rtol=0, atol=1e-9), i


def pin_rms_scale_invariance(o):
    """With eps = 0, scaling X by 2^k (exact) leaves the maps unchanged and
    scales h by 2^k."""
    rng = np.random.default_rng(22)
    X, phi, bias, _, _ = _layer_inputs(rng, 3, 4, 8, (1.0, 1.0, 1.0))
    al = (1.0, 1.0, 1.0)
    a = o.pre(X, phi, bias, al, eps=0.0)
    b = o.pre((X * np.float32(8.0)).astype(np.float32), phi, bias, al, eps=0.0)
    assert np.allclose(a["H"], b["H"], rtol=1e-14, atol=1e-15)
    assert np.allclose(8.0 * a["h"], b["h"], rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# Storage rounding and the stack workload's sublayer.

def pin_bf16_rounding(o):
    """Round to nearest, ties to even, at bf16's 8-bit significand."""
    cases = [
        (1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82), (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),
        (-2.0, 0xC000), (0.0, 0x0000), (3.0e38, 0x7F62), (1e39, 0x7F80),
        (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),             # subnormal quantum, tie -> 0
    ]
    got = o.round_bf16([c[0] for c in cases])
    for (v, bits), g in zip(cases, got):
        assert int(g) == bits, (v, hex(int(g)), hex(bits))


def pin_gelu_half(o):
    """0.5 GELU(h) = 0.5 h Phi(h): Phi(0) = 1/2, Phi(1) = 0.841344746068543,
    Phi(-1) = 0.158655253931457 (standard normal CDF)."""
    h = np.array([0.0, 1.0, -1.0, 2.0], dtype=np.float32)
    y = o.gelu_half(h)
    assert y[0] == 0.0
    assert abs(y[1] - 0.5 * 0.841344746068543) <= 1e-15
    assert abs(y[2] - 0.5 * -1.0 * 0.158655253931457) <= 1e-15
    assert abs(y[3] - 0.5 * 2.0 * 0.977249868051821) <= 1e-15


def pin_stack_matches_layers(o):
    """The stack's first two layers equal pre -> round -> 0.5 GELU -> round ->
    post -> round, done step by step with the single-layer functions."""
    rng = np.random.default_rng(23)
    n, d, T, L = 4, 8, 3, 2
    X0 = rng.normal(0, 1, (T, n, d)).astype(np.float32)
    bits = o.round_bf16(X0.astype(np.float64))
    phis = rng.normal(0, 0.3, (L, n * d, 24)).astype(np.float32)
    biases = rng.normal(0, 0.5, (L, 24)).astype(np.float32)
    alphas = np.full((L, 3), 0.5, np.float32)
    st = o.stack(bits, phis, biases, alphas)
    X = bits
    for l in range(L):
        out = o.pre(X, phis[l], biases[l], alphas[l])
        Hf = out["H"].astype(np.float32)
        assert np.array_equal(st["H"][l], Hf)
        hb = o.round_bf16(out["h"])
        yb = o.round_bf16(o.gelu_half(hb))
        X = o.round_bf16(o.post(X, yb, Hf))
    assert np.array_equal(st["X"], X)
    am = o.amax(st["H"], n)
    assert np.array_equal(am["amax"], st["amax"])


# --------------------------------------------------------------------------
# Backward.  The pages give no backward formulas, only that the layer trains
# with a custom backward that recomputes the maps ([P5] mixed-precision table
# and kernel notes); the oracle's backward is the chain rule of its forward.
# It is pinned by central finite differences of the all-double forward and by
# exact identities of the forward.  The differentiated quantity is
# L = sum_t <G_t, X'_t> + <D_t, h_t> with G and D given.

def _bwd_inputs(rng, T, n, d, alpha):
    X, phi, bias, al, Y = _layer_inputs(rng, T, n, d, alpha)
    G = rng.normal(0.0, 1.0, (T, n, d)).astype(np.float32)
    D = rng.normal(0.0, 1.0, (T, d)).astype(np.float32)
    return X, Y, phi, bias, al, G, D


def _loss(o, X, Y, phi, bias, al, G, D, eps, t_max):
    h, Xo = o.layer_f64(X, Y, phi, bias, al, eps=eps, t_max=t_max)
    return float(np.sum(G.astype(np.float64) * Xo) + np.sum(D.astype(np.float64) * h))


def _fd_check(o, args, which, idx, analytic, eps, t_max, step, rtol, atol):
    """Central differences of L in the coordinates ``idx`` of argument ``which``."""
    base = [np.array(a, dtype=np.float64) for a in args]
    worst = 0.0
    for flat in idx:
        plus = [a.copy() for a in base]
        minus = [a.copy() for a in base]
        plus[which].reshape(-1)[flat] += step
        minus[which].reshape(-1)[flat] -= step
        fd = (_loss(o, *plus, eps=eps, t_max=t_max) - _loss(o, *minus, eps=eps, t_max=t_max)) / (2.0 * step)
        an = float(np.asarray(analytic).reshape(-1)[flat])
        err = abs(fd - an)
        worst = max(worst, err / (atol + rtol * abs(an)))
        assert err <= atol + rtol * abs(an), (which, flat, fd, an)
    return worst


def pin_bwd_finite_differences(o):
    """Every gradient (X, Y, phi, bias, alpha) against central differences of
    the all-double forward, on a T = 8, n = 4, d = 32 slice of the layer
    workload's distributions, at the workload's alpha and at a large alpha
    that makes the projection, gates and Sinkhorn matter."""
    rng = np.random.default_rng(31)
    T, n, d = 8, 4, 32
    m = n * n + 2 * n
    for alpha in ((0.01, 0.01, 0.01), (1.0, 0.7, -0.4)):
        X, Y, phi, bias, al, G, D = _bwd_inputs(rng, T, n, d, alpha)
        g = o.bwd_f64(X, Y, phi, bias, al, G, D, eps=1e-6, t_max=20)
        args = (X, Y, phi, bias, al, G, D)
        pick = lambda size, k: rng.choice(size, size=min(k, size), replace=False)
        # X: 48 coordinates spread over tokens and streams; Y: 16
        _fd_check(o, args, 0, pick(T * n * d, 48), g["dX"], 1e-6, 20, 1e-5, 1e-6, 1e-8)
        _fd_check(o, args, 1, pick(T * d, 16), g["dY"], 1e-6, 20, 1e-5, 1e-6, 1e-8)
        # phi: two entries of every column
        cols = np.repeat(np.arange(m), 2)
        rows = rng.integers(0, n * d, cols.size)
        _fd_check(o, args, 2, rows * m + cols, g["dphi"], 1e-6, 20, 1e-5, 1e-6, 1e-8)
        _fd_check(o, args, 3, np.arange(m), g["dbias"], 1e-6, 20, 1e-5, 1e-6, 1e-8)
        _fd_check(o, args, 4, np.arange(3), g["dalpha"], 1e-6, 20, 1e-6, 1e-6, 1e-8)


def pin_bwd_single_token_logits(o):
    """With one token the bias gradient is that token's logit gradient, so
    central differences in the bias pin dlogit (and through it dH) per token,
    also after a single Sinkhorn pass and with no pass at all."""
    rng = np.random.default_rng(32)
    n, d = 3, 5
    for t_max in (0, 1, 20):
        X, Y, phi, bias, al, G, D = _bwd_inputs(rng, 1, n, d, (0.8, 1.3, -0.6))
        g = o.bwd_f64(X, Y, phi, bias, al, G, D, eps=1e-6, t_max=t_max)
        assert np.array_equal(g["dlogit"][0], g["dbias"])
        _fd_check(o, (X, Y, phi, bias, al, G, D), 3, np.arange(n * n + 2 * n), g["dbias"], 1e-6, t_max,
                  1e-5, 1e-6, 1e-8)


def pin_bwd_column_shift_invariance(o):
    """Adding a constant to one column of the residual logits scales that
    column of exp(.) and is undone exactly by the first column normalisation,
    so each column of dL/dlogits_res sums to zero (row shifts are not exact)."""
    rng = np.random.default_rng(33)
    T, n, d = 4, 4, 16
    X, Y, phi, bias, al, G, D = _bwd_inputs(rng, T, n, d, (1.0, 1.0, 1.0))
    for t_max in (1, 20):
        g = o.bwd_f64(X, Y, phi, bias, al, G, D, t_max=t_max)
        dres = g["dlogit"][:, n:n + n * n].reshape(T, n, n)
        scale = np.max(np.abs(dres))
        assert scale > 1e-3
        assert np.max(np.abs(dres.sum(axis=1))) <= 1e-13 * scale, dres.sum(axis=1)
        if t_max == 1:      # one pass is far from converged: row shifts do change the result
            assert np.max(np.abs(dres.sum(axis=2))) > 1e-3 * scale


def pin_bwd_alpha0_closed_form(o):
    """alpha = 0: the maps do not depend on X, so dX_j = sum_i H_res[i][j] G_i
    + sigmoid(b_pre,j) D and dY = sum_i 2 sigmoid(b_post,i) G_i with
    H_res = SK(exp(b_res)); dphi = 0; dH_res[i][j] = <G_i, X_j>,
    dH_post[i] = <G_i, Y>, dH_pre[i] = <D, X_i>."""
    rng = np.random.default_rng(34)
    T, n, d = 3, 4, 8
    X, Y, phi, bias, _, G, D = _bwd_inputs(rng, T, n, d, (0.0, 0.0, 0.0))
    g = o.bwd_f64(X, Y, phi, bias, (0.0, 0.0, 0.0), G, D)
    b = bias.astype(np.float64)
    Hres = o.sinkhorn(b[n:n + n * n].reshape(n, n), 20)
    spre = 1.0 / (1.0 + np.exp(-b[:n]))
    wpost = 2.0 / (1.0 + np.exp(-b[n + n * n:]))
    Xd, Gd, Yd, Dd = (a.astype(np.float64) for a in (X, G, Y, D))
    for t in range(T):
        assert np.allclose(g["dX"][t], Hres.T @ Gd[t] + spre[:, None] * Dd[t][None, :], rtol=1e-13, atol=1e-14)
        assert np.allclose(g["dY"][t], wpost @ Gd[t], rtol=1e-13, atol=1e-14)
        assert np.allclose(g["dH"][t, n:n + n * n].reshape(n, n), Gd[t] @ Xd[t].T, rtol=1e-13, atol=1e-13)
        assert np.allclose(g["dH"][t, n + n * n:], Gd[t] @ Yd[t], rtol=1e-13, atol=1e-13)
        assert np.allclose(g["dH"][t, :n], Xd[t] @ Dd[t], rtol=1e-13, atol=1e-13)
    assert np.all(g["dphi"] == 0.0)


def pin_bwd_euler_homogeneity(o):
    """With eps = 0 the maps are invariant to scaling X, so h and X' - H_post Y
    are homogeneous of degree 1 in X (Euler): sum x . dx equals
    sum_t <G_t, H_res X_t> + <D_t, h_t>, i.e. the RMSNorm path's share of dx
    is orthogonal to x."""
    rng = np.random.default_rng(35)
    T, n, d = 3, 4, 8
    X, Y, phi, bias, _, G, D = _bwd_inputs(rng, T, n, d, (1.0, 1.0, 1.0))
    al = (1.5, 0.8, -1.1)
    g = o.bwd_f64(X, Y, phi, bias, al, G, D, eps=0.0)
    h, Xo = o.layer_f64(X, np.zeros_like(Y), phi, bias, al, eps=0.0)
    lhs = float(np.sum(X.astype(np.float64) * g["dX"]))
    rhs = float(np.sum(G.astype(np.float64) * Xo) + np.sum(D.astype(np.float64) * h))
    assert abs(lhs - rhs) <= 1e-11 * (abs(rhs) + 1.0), (lhs, rhs)


def pin_bwd_storage_forms_agree(o):
    """The storage-typed backward (fp32 and bf16 state, any token list) gives
    the all-double backward's values on the same numbers; parameter gradients
    add over disjoint token lists."""
    rng = np.random.default_rng(36)
    T, n, d = 5, 4, 8
    X, Y, phi, bias, al, G, D = _bwd_inputs(rng, T, n, d, (0.5, 0.5, 0.5))
    ref = o.bwd_f64(X, Y, phi, bias, al, G, D)
    got = o.bwd(X, Y, phi, bias, al, G, D)
    for k in ref:
        assert np.allclose(got[k], ref[k], rtol=1e-14, atol=1e-15), k
    bits = [o.round_bf16(a.astype(np.float64)) for a in (X, Y, G, D)]
    vals = [(b.astype(np.uint32) << 16).view(np.float32) for b in bits]
    refb = o.bwd_f64(vals[0], vals[1], phi, bias, al, vals[2], vals[3])
    gotb = o.bwd(bits[0], bits[1], phi, bias, al, bits[2], bits[3])
    for k in refb:
        assert np.allclose(gotb[k], refb[k], rtol=1e-14, atol=1e-15), k
    a = o.bwd(X, Y, phi, bias, al, G, D, tokens=[4, 1])
    b = o.bwd(X, Y, phi, bias, al, G, D, tokens=[0, 2, 3])
    assert np.allclose(a["dX"], ref["dX"][[4, 1]], rtol=1e-15, atol=0)
    for k in ("dphi", "dbias", "dalpha"):
        assert np.allclose(a[k] + b[k], ref[k], rtol=1e-12, atol=1e-15), k


# --------------------------------------------------------------------------
# The HC form of the maps, for contrast ([P2] Kernmechanismen: a static bias
# plus an input-dependent term through tanh, either sign; reading
# H = bias + alpha_blk * tanh(z), no Sinkhorn).

def pin_hc_maps_closed_form(o):
    """One-hot phi columns give z exactly (as for mHC), so every map is
    bias + alpha_blk * tanh(c / r); alpha = 0 leaves the bias itself, which
    for HC is the map (no exp, no normalisation, no gate)."""
    n, d, m = 4, 8, 24
    rng = np.random.default_rng(40)
    X = rng.normal(0, 1, (1, n, d)).astype(np.float32)
    x = X.reshape(-1).astype(np.float64)
    r = math.sqrt(float(np.mean(x * x)) + 1e-6)
    phi = np.zeros((n * d, m), dtype=np.float32)
    for j in range(m):
        phi[(5 * j) % (n * d), j] = 1.0
    bias = rng.normal(0, 0.5, m).astype(np.float32)
    alpha = (0.7, -1.3, 2.1)
    H = o.pre_hc(X, phi, bias, alpha)["H"][0]
    for j in range(m):
        a = float(np.float32(alpha[0] if j < n else alpha[1] if j < n + n * n else alpha[2]))
        expect = float(bias[j]) + a * math.tanh(x[(5 * j) % (n * d)] / r)
        assert abs(H[j] - expect) <= 1e-12, (j, H[j], expect)
    H0 = o.pre_hc(X, phi, bias, (0.0, 0.0, 0.0))
    assert np.array_equal(H0["H"][0], bias.astype(np.float64))
    assert np.allclose(H0["h"][0], bias[:n].astype(np.float64) @ X[0].astype(np.float64), rtol=1e-14, atol=1e-14)


def pin_hc_odd_and_bounded(o):
    """tanh is odd and bounded: H(phi) + H(-phi) = 2 bias, |H - bias| < |alpha|,
    and the residual map is not normalised (its rows do not sum to one)."""
    rng = np.random.default_rng(41)
    X, phi, bias, _, _ = _layer_inputs(rng, 5, 4, 16, (1.0, 1.0, 1.0), bres=1.0)
    phi = (phi * 50).astype(np.float32)                 # large z: tanh saturates
    alpha = (0.5, 0.8, -0.6)
    a = o.pre_hc(X, phi, bias, alpha)["H"]
    b = o.pre_hc(X, (-phi).astype(np.float32), bias, alpha)["H"]
    assert np.allclose(a + b, 2.0 * bias.astype(np.float64)[None, :], rtol=0, atol=1e-14)
    lim = np.concatenate([np.full(4, 0.5), np.full(16, 0.8), np.full(4, 0.6)]).astype(np.float32)
    assert np.all(np.abs(a - bias.astype(np.float64)[None, :]) <= lim.astype(np.float64)[None, :])
    rows = a[:, 4:20].reshape(5, 4, 4).sum(axis=2)
    assert np.max(np.abs(rows - 1.0)) > 0.1


def pin_hc_stack_compounds(o):
    """The pages' point about the composite map: with every residual map
    1.1 I (alpha = 0, bias only) the product over 60 layers is 1.1^60 I, an
    Amax of 1.1^60 ~ 304 (the pages' ~300), and with zero read and write
    maps the state itself is scaled by 1.1^60.  The mHC form of the same
    bias is doubly stochastic: Amax 1 (to Sinkhorn's 20-pass accuracy)."""
    n, d, T, L = 4, 8, 3, 60
    rng = np.random.default_rng(42)
    X0 = rng.normal(0, 1, (T, n, d)).astype(np.float32)
    phis = rng.normal(0, 0.02, (L, n * d, 24)).astype(np.float32)
    biases = np.zeros((L, 24), np.float32)
    biases[:, 4:20] = (1.1 * np.eye(n)).reshape(-1)
    biases[:, :4] = 0.0                                  # HC read map 0: h = 0, F(0) = 0
    biases[:, 20:] = 0.0                                 # HC write map 0
    alphas = np.zeros((L, 3), np.float32)
    g = float(np.float32(1.1)) ** 60                     # the bias is stored in fp32
    hc = o.stack_hc(X0, phis, biases, alphas)
    assert np.allclose(hc["amax"], g, rtol=1e-12), hc["amax"]
    assert abs(g - 304.48) < 0.01
    assert np.allclose(hc["X"].astype(np.float64), g * X0.astype(np.float64), rtol=1e-5, atol=0)
    mhc = o.stack(X0, phis, biases, alphas)              # doubly stochastic to Sinkhorn's 20-pass accuracy
    assert np.all(np.abs(mhc["amax"] - 1.0) < 1e-5), mhc["amax"]


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
