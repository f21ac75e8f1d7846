"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Same seeded inputs on both sides; the oracle computes in double from the
exact stored inputs.  Every case compares every output element; at full size
the oracle runs over token chunks on host threads (it computes each token on
its own).
"""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL, assert_close, check_stack_every_token, dname, for_token_chunks, to_device, to_host, values

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


def _layer(mhc, o, w, T=None, alpha=None, tokens=None, inplace=False, check_post=True):
    """Run one layer on the GPU and the oracle; compare h, H and X'."""
    T = w.T if T is None else T
    alpha = w.alpha if alpha is None else alpha
    X = synth.make_state(w, T)
    Y = synth.make_sublayer_out(w, T)
    phi, bias = synth.make_params(w)
    dX, dY = to_device(X), to_device(Y)
    dphi, dbias = to_device(phi), to_device(bias)
    h, H = mhc.pre(dX, dphi, dbias, alpha=alpha, eps=w.eps, t_max=w.t_max)
    Hh = to_host(H)
    Xo = mhc.post(dX, dY, H, out=dX if inplace else None)
    torch.cuda.synchronize()
    tok = np.arange(T, dtype=np.int64) if tokens is None else tokens
    ref = o.pre(X, phi, bias, alpha, eps=w.eps, t_max=w.t_max, tokens=tok)
    dn = dname(w.dtype)
    assert_close(Hh[tok], ref["H"], *TOL[(dn, "maps")], what=f"{w.name} H")
    assert_close(to_host(h)[tok], ref["h"], *TOL[(dn, "state")], what=f"{w.name} h")
    if check_post:
        # X' from the GPU's own maps, and also X' of the oracle maps checked
        # end to end: the oracle's post consumes the oracle's fp32 maps.
        Xo_ref = o.post(X, Y, ref["H"].astype(np.float32), tokens=tok)
        assert_close(to_host(Xo)[tok], Xo_ref, *TOL[(dn, "state")], what=f"{w.name} X'")
    return Hh, to_host(h), to_host(Xo)


SMALL = [
    ("layer_fp32_T64_d256", {}),
    ("layer_bf16_T4096_d2048", {"T": 200}),
    ("layer_bf16_T16384_d4096", {"T": 130}),
    ("stack60_bf16_T4096_d2560", {"T": 70, "layers": 1, "sublayer": "given"}),
]


@pytest.mark.parametrize("name,changes", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("alpha", [None, (1.0, 1.0, 1.0)], ids=["alpha_cfg", "alpha_1"])
def test_layer_every_token(mhc, oracle_lib, name, changes, alpha):
    """All tokens of reduced-T versions of the workloads (several tiles and a
    ragged tail), at the workloads' alpha and at alpha = 1, where the
    projection is not damped 100x."""
    w = synth.scaled(synth.WORKLOADS[name], **changes)
    _layer(mhc, oracle_lib, w, alpha=alpha)


PERSISTENT = [
    # (n, d, T): enough tokens for the persistent two-pass form (ceil(T / 32) * ceil(d / 256) >= 128),
    # whose bf16 tiles go through LDS; ragged slices of d and ragged last tiles
    (4, 2056, 600),
    (2, 264, 2100),
    (1, 4096, 300),
    (4, 1024, 1100),
]


@pytest.mark.parametrize("n,d,T", PERSISTENT, ids=[f"n{c[0]}_d{c[1]}_T{c[2]}" for c in PERSISTENT])
def test_two_pass_persistent_every_token(mhc, oracle_lib, n, d, T):
    """The persistent two-pass mhc_pre (LDS-staged bf16 tiles) against the
    oracle on every token, at alpha = 1."""
    w = synth.Workload(f"persist_n{n}_d{d}", T=T, n=n, d=d, dtype=synth.BF16, seed=6100 + n + d)
    X = synth.make_state(w)
    phi, bias = synth.make_params(w)
    alpha = (1.0, 1.0, 1.0)
    h, H, used = mhc.pre_ex(to_device(X), to_device(phi), to_device(bias), mhc.PRE_TWO_PASS, alpha=alpha,
                            eps=w.eps, t_max=w.t_max)
    torch.cuda.synchronize()
    assert used == mhc.PRE_TWO_PASS
    ref = oracle_lib.pre(X, phi, bias, alpha, eps=w.eps, t_max=w.t_max)
    assert_close(to_host(H), ref["H"], *TOL[("bf16", "maps")], what=f"{w.name} H")
    assert_close(to_host(h), ref["h"], *TOL[("bf16", "state")], what=f"{w.name} h")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["layer_bf16_T4096_d2048", "layer_bf16_T16384_d4096"])
def test_layer_full_size_every_token(mhc, oracle_lib, name):
    """The full-size workloads in the benchmark's launch configuration
    (mhc_pre as MHC_PRE_AUTO picks it, then mhc_post), checked on every token:
    h, H and X' (the GPU's X' from its own maps, and the oracle's X' from the
    oracle's maps)."""
    w = synth.WORKLOADS[name]
    print(f"[parity] full size {name}", flush=True)
    X, Y = synth.make_state(w), synth.make_sublayer_out(w)
    phi, bias = synth.make_params(w)
    dX, dY = to_device(X), to_device(Y)
    h, H = mhc.pre(dX, to_device(phi), to_device(bias), alpha=w.alpha, eps=w.eps, t_max=w.t_max)
    Xo = mhc.post(dX, dY, H)
    torch.cuda.synchronize()
    Hh, hh, Xoh = to_host(H), to_host(h), to_host(Xo)
    del dX, dY, h, H, Xo
    dn = dname(w.dtype)

    def cmp(tok):
        ref = oracle_lib.pre(X, phi, bias, w.alpha, eps=w.eps, t_max=w.t_max, tokens=tok)
        assert_close(Hh[tok], ref["H"], *TOL[(dn, "maps")], what=f"{w.name} H, tokens {tok[0]}..")
        assert_close(hh[tok], ref["h"], *TOL[(dn, "state")], what=f"{w.name} h, tokens {tok[0]}..")
        Xo_ref = oracle_lib.post(X, Y, ref["H"].astype(np.float32), tokens=tok)
        assert_close(Xoh[tok], Xo_ref, *TOL[(dn, "state")], what=f"{w.name} X', tokens {tok[0]}..")

    for_token_chunks(cmp, w.T)


# d = 512 and 1536: multiples of 512, where mhc_post takes its tiled kernel (4-token tiles; T = 3 and 9
# leave a partial last tile).
EDGE = [(n, d, T, dt) for n in (1, 2, 4)
        for (d, T) in ((8, 1), (24, 17), (264, 65), (520, 33), (2048 + 8, 5), (512, 3), (1536, 9))
        for dt in (synth.FP32, synth.BF16)]


@pytest.mark.parametrize("n,d,T,dt", EDGE, ids=[f"n{e[0]}_d{e[1]}_T{e[2]}_{dname(e[3])}" for e in EDGE])
def test_edge_shapes(mhc, oracle_lib, n, d, T, dt):
    """Streams 1/2/4, d below one slice and with ragged slices, T = 1 and T
    not a multiple of the token tile, both storage types, alpha = 1."""
    w = synth.Workload(f"edge_n{n}_d{d}", T=T, n=n, d=d, dtype=dt, seed=4242 + n * 7 + d)
    _layer(mhc, oracle_lib, w, alpha=(1.0, 0.5, -0.75))


def test_post_in_place(mhc, oracle_lib):
    """X' written over X (the exact alias the ABI allows)."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T4096_d2048"], T=96)
    _layer(mhc, oracle_lib, w, inplace=True)


def test_bitwise_deterministic(mhc):
    """Two runs on the same inputs give identical bits (fixed-order reductions)."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=300)
    X = to_device(synth.make_state(w))
    Y = to_device(synth.make_sublayer_out(w))
    phi, bias = (to_device(a) for a in synth.make_params(w))
    outs = []
    for _ in range(2):
        h, H = mhc.pre(X, phi, bias, alpha=w.alpha)
        Xo = mhc.post(X, Y, H)
        torch.cuda.synchronize()
        outs.append((to_host(h), to_host(H), to_host(Xo)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_zero_tokens_is_noop(mhc):
    X = torch.empty((0, 4, 256), dtype=torch.bfloat16, device="cuda")
    phi = torch.zeros((1024, 24), device="cuda")
    bias = torch.zeros(24, device="cuda")
    h, H = mhc.pre(X, phi, bias)
    assert h.shape == (0, 256) and H.shape == (0, 24)


def test_equal_streams_pass_through(mhc):
    """Identical streams and Y = 0: rows of H_res sum to 1, so X' = X up to
    the bf16 rounding of the output."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T4096_d2048"], T=64)
    x = synth.normal(w.seed, 99, (w.T, 1, w.d), dtype=synth.BF16)
    X = np.repeat(x, w.n, axis=1)
    phi, bias = synth.make_params(w)
    dX = to_device(X)
    h, H = mhc.pre(dX, to_device(phi), to_device(bias), alpha=w.alpha)
    Xo = mhc.post(dX, torch.zeros((w.T, w.d), dtype=torch.bfloat16, device="cuda"), H)
    torch.cuda.synchronize()
    assert_close(to_host(Xo), values(X), 4e-3, 1e-6, what="equal streams")


@pytest.mark.parametrize("n", [1, 2, 4])
@pytest.mark.parametrize("L", [0, 1, 7, 60])
def test_amax_matches_oracle(mhc, oracle_lib, n, L):
    """Composite Amax of random (not doubly stochastic) maps and of Sinkhorn maps."""
    T = 300
    m = n * n + 2 * n
    rng = np.random.default_rng(100 + n * 10 + L)
    Hs = (np.eye(n).reshape(1, 1, -1) + 0.3 * rng.standard_normal((L, T, n * n)))
    Hfull = np.zeros((L, T, m), np.float32)
    Hfull[:, :, n:n + n * n] = Hs
    dH = to_device(Hfull)
    r = mhc.amax(dH, n)
    torch.cuda.synchronize()
    ref = oracle_lib.amax(Hfull, n)
    for k in ("amax", "gain_fwd", "gain_bwd"):
        assert_close(to_host(r[k]), ref[k], 1e-4, 1e-6, what=f"amax {k}")
    scale = np.abs(ref["composite"]).max(axis=(1, 2), keepdims=True)   # products of random maps cancel
    err = np.abs(to_host(r["composite"]) - ref["composite"])
    assert np.all(err <= 1e-4 * scale + 1e-6), float((err / scale).max())


@pytest.mark.parametrize("count", [7, 1003, 24581])
def test_gelu_half(mhc, oracle_lib, count):
    """Fewer values than one 8-value chunk, a ragged tail, and several
    workgroups of 512 chunks with a ragged tail."""
    for dt in (synth.FP32, synth.BF16):
        h = synth.normal(5, 1, (count,), 0.0, 2.0, dt)
        y = to_host(mhc.gelu_half(to_device(h)))
        tol = (1e-5, 1e-6) if dt == synth.FP32 else (8e-3, 1e-6)
        assert_close(y, oracle_lib.gelu_half(h), *tol, what="gelu_half")


def test_gelu_half_extremes(mhc, oracle_lib):
    """Values far in both tails (the 60-layer stack's state reaches ~1e18),
    where 1 + erf(h / sqrt 2) cancels for negative h, plus +-inf and NaN, which
    propagate as in the oracle.  The oracle forms 1 + erf in double, whose
    absolute error near erf = -1 is up to 2^-53 (from h ~ -8.3 on it returns
    0 where the value is ~1e-19): the bound adds 0.25 |h| 2^-52 for that."""
    big = [-1e30, -1e18, -1e4, -20.0, -12.0, -9.0, -5.5, -5.0, -4.0, -3.0, -1.0, -1e-3, -0.0, 0.0, 1e-3, 1.0, 3.0, 5.0,
           9.0, 20.0, 1e4, 1e18, 1e30]
    for dt in (synth.FP32, synth.BF16):
        f = np.array(big, np.float64)
        h = f.astype(np.float32) if dt == synth.FP32 else oracle_lib.round_bf16(f)
        hv = h.astype(np.float64) if dt == synth.FP32 else synth.bf16_bits_to_f32(h).astype(np.float64)
        y = to_host(mhc.gelu_half(to_device(h)))
        yv = y.astype(np.float64) if dt == synth.FP32 else synth.bf16_bits_to_f32(y).astype(np.float64)
        ref = oracle_lib.gelu_half(h)
        rtol = 2e-5 if dt == synth.FP32 else 8e-3
        bound = rtol * np.abs(ref) + 0.25 * np.abs(hv) * 2.0 ** -52 + 1e-30
        assert np.all(np.abs(yv - ref) <= bound), (dt, hv[np.abs(yv - ref) > bound], yv[np.abs(yv - ref) > bound],
                                                   ref[np.abs(yv - ref) > bound])
        s = np.array([np.inf, -np.inf, np.nan], np.float64)
        hs = s.astype(np.float32) if dt == synth.FP32 else oracle_lib.round_bf16(s)
        ys = to_host(mhc.gelu_half(to_device(hs)))
        ys = synth.bf16_bits_to_f32(ys) if dt == synth.BF16 else ys
        ref = oracle_lib.gelu_half(hs)
        assert ys[0] == np.inf and ref[0] == np.inf
        assert np.isnan(ys[1]) and np.isnan(ref[1])      # -inf * 0 in both
        assert np.isnan(ys[2]) and np.isnan(ref[2])


def _stack(mhc, w, T, L):
    """L layers of pre -> 0.5 GELU -> post on the GPU; returns X_L and the maps."""
    X0 = synth.make_state(w, T)
    phis, biases = zip(*(synth.make_params(w, layer=l) for l in range(L)))
    X = to_device(X0)
    Hs = torch.empty((L, T, w.m), dtype=torch.float32, device="cuda")
    for l in range(L):
        h, _ = mhc.pre(X, to_device(phis[l]), to_device(biases[l]), alpha=w.alpha, eps=w.eps, t_max=w.t_max,
                       H=Hs[l])
        Y = mhc.gelu_half(h)
        X = mhc.post(X, Y, Hs[l])
    am = mhc.amax(Hs, w.n)
    torch.cuda.synchronize()
    return X0, np.stack(phis), np.stack(biases), to_host(X), to_host(Hs), {k: to_host(v) for k, v in am.items()}


@pytest.mark.parametrize("T,L", [(40, 60), (4096, 60)], ids=["T40", "T4096"])
def test_stack60(mhc, oracle_lib, T, L):
    """The 60-layer stack: final state, every layer's maps and the composite
    Amax per token (within 1e-3 relative of the oracle's), on every token."""
    w = synth.WORKLOADS["stack60_bf16_T4096_d2560"]
    print(f"[parity] stack T={T} L={L}", flush=True)
    X0, phis, biases, Xg, Hg, am = _stack(mhc, w, T, L)
    check_stack_every_token(oracle_lib, w, X0, phis, biases, Xg, Hg, am, L)
