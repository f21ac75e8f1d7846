"""n = 8 streams: mhc_pre (its own split-K kernels: 80 maps per token, a
64-entry Sinkhorn-Knopp on one wave per token), mhc_post, mhc_post_pre and
mhc_amax against the oracle.

Shapes cover d below one 512-position slice, ragged last slices, T = 1 and T
not a multiple of the 16-token tile, both storage types, both map forms; one
case runs at d = 4096 with enough tokens for several persistent passes, and
one at the benchmark's n = 8 shape (T = 16384, d = 4096), every token.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL, assert_close, dname, for_token_chunks, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


CASES = [
    # (d, T, dtype)
    (8, 1, synth.FP32),
    (64, 17, synth.BF16),
    (264, 65, synth.BF16),      # one 264-position slice per stream
    (520, 33, synth.FP32),      # a full slice and an 8-position one per stream
    (1024, 130, synth.BF16),
    (4096, 700, synth.BF16),    # 64 slices; 22 tiles over more workgroup passes than one
]


def _inputs(d, T, dtype, seed):
    w = synth.Workload(f"n8_d{d}_T{T}", T=T, n=8, d=d, dtype=dtype, seed=seed)
    return w, synth.make_state(w), synth.make_sublayer_out(w), synth.make_params(w)


@pytest.mark.parametrize("d,T,dtype", CASES, ids=[f"d{c[0]}_T{c[1]}_{dname(c[2])}" for c in CASES])
@pytest.mark.parametrize("maps", ["mhc", "hc"])
def test_n8_layer_every_token(mhc, oracle_lib, d, T, dtype, maps):
    w, X, Y, (phi, bias) = _inputs(d, T, dtype, 5100 + d + T)
    alpha = (1.0, 0.5, -0.75)
    code = mhc.MAPS_HC if maps == "hc" else mhc.MAPS_MHC
    dX, dY = to_device(X), to_device(Y)
    h, H = mhc.pre(dX, to_device(phi), to_device(bias), alpha=alpha, eps=w.eps, t_max=w.t_max, maps=code)
    Xo = mhc.post(dX, dY, H)
    torch.cuda.synchronize()
    dn = dname(dtype)
    rtol, atol = TOL[(dn, "maps")]
    if maps == "hc":
        ref = oracle_lib.pre_hc(X, phi, bias, alpha, eps=w.eps)
        atol = atol * max(1.0, 4.0 * max(abs(a) for a in alpha))
    else:
        ref = oracle_lib.pre(X, phi, bias, alpha, eps=w.eps, t_max=w.t_max)
    assert_close(to_host(H), ref["H"], rtol, atol, what=f"{w.name} {maps} H")
    assert_close(to_host(h), ref["h"], *TOL[(dn, "state")], what=f"{w.name} {maps} h")
    Xo_ref = oracle_lib.post(X, Y, to_host(H))
    assert_close(to_host(Xo), Xo_ref, *TOL[(dn, "state")], what=f"{w.name} {maps} X'")


def test_n8_full_size_every_token(mhc, oracle_lib):
    """The benchmark's n = 8 shape (T = 16384, d = 4096, bf16: 1 GiB of state,
    64 slices of 512 positions, many persistent passes), the workloads'
    distributions: h, H and X' of every token against the oracle."""
    w = synth.Workload("n8_T16384_d4096", T=16384, n=8, d=4096, dtype=synth.BF16, seed=5901)
    print(f"[parity] full size {w.name}", flush=True)
    X, Y = synth.make_state(w), synth.make_sublayer_out(w)
    phi, bias = synth.make_params(w)
    dX, dY = to_device(X), to_device(Y)
    h, H = mhc.pre(dX, to_device(phi), to_device(bias), alpha=w.alpha, eps=w.eps, t_max=w.t_max)
    Xo = mhc.post(dX, dY, H)
    torch.cuda.synchronize()
    Hh, hh, Xoh = to_host(H), to_host(h), to_host(Xo)
    del dX, dY, h, H, Xo

    def cmp(tok):
        ref = oracle_lib.pre(X, phi, bias, w.alpha, eps=w.eps, t_max=w.t_max, tokens=tok)
        assert_close(Hh[tok], ref["H"], *TOL[("bf16", "maps")], what=f"{w.name} H, tokens {tok[0]}..")
        assert_close(hh[tok], ref["h"], *TOL[("bf16", "state")], what=f"{w.name} h, tokens {tok[0]}..")
        Xo_ref = oracle_lib.post(X, Y, ref["H"].astype(np.float32), tokens=tok)
        assert_close(Xoh[tok], Xo_ref, *TOL[("bf16", "state")], what=f"{w.name} X', tokens {tok[0]}..")

    for_token_chunks(cmp, w.T)


def test_n8_sinkhorn_is_doubly_stochastic(mhc, oracle_lib):
    """Strong residual logits (alpha = 1, large diagonal bias): after the
    last row step every row of H_res sums to 1 to fp32 rounding; 20 passes
    leave a column residual, which must be the oracle's."""
    w, X, _, (phi, bias) = _inputs(512, 64, synth.BF16, 5200)
    bias = bias.copy()
    bias[8:72] += (4.0 * np.eye(8)).reshape(-1).astype(np.float32)
    h, H = mhc.pre(to_device(X), to_device(phi), to_device(bias), alpha=(1.0, 1.0, 1.0))
    torch.cuda.synchronize()
    R = to_host(H)[:, 8:72].astype(np.float64).reshape(-1, 8, 8)
    ref = oracle_lib.pre(X, phi, bias, (1.0, 1.0, 1.0))["H"][:, 8:72].reshape(-1, 8, 8)
    assert np.all(R > 0)
    assert np.max(np.abs(R.sum(axis=2) - 1.0)) < 1e-5
    assert np.max(np.abs(R.sum(axis=1) - ref.sum(axis=1))) < 1e-4


def test_n8_post_pre_matches_separate_calls(mhc):
    """At n = 8 mhc_post_pre runs the two entry points one after the other:
    identical bits to calling them separately."""
    w, X, Y, (phi, bias) = _inputs(1024, 100, synth.BF16, 5300)
    dX, dY = to_device(X), to_device(Y)
    dphi, dbias = to_device(phi), to_device(bias)
    _, H0 = mhc.pre(dX, dphi, dbias, alpha=(0.5, 0.5, 0.5))
    Xf, hf, Hf = mhc.post_pre(dX, dY, H0, dphi, dbias, alpha=(0.7, 0.3, 0.2))
    Xs = mhc.post(dX, dY, H0)
    hs, Hs = mhc.pre(Xs, dphi, dbias, alpha=(0.7, 0.3, 0.2))
    torch.cuda.synchronize()
    for a, b in ((Xf, Xs), (hf, hs), (Hf, Hs)):
        assert np.array_equal(to_host(a), to_host(b))


def test_n8_bitwise_deterministic(mhc):
    w, X, _, (phi, bias) = _inputs(2048, 300, synth.BF16, 5400)
    dX, dphi, dbias = to_device(X), to_device(phi), to_device(bias)
    outs = []
    for _ in range(2):
        h, H = mhc.pre(dX, dphi, dbias, alpha=(1.0, 1.0, 1.0))
        torch.cuda.synchronize()
        outs.append((to_host(h), to_host(H)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_n8_one_pass_is_refused(mhc):
    """The single-pass form covers n <= 4: asking for it at n = 8 is an
    error, and AUTO takes the two-pass form."""
    w, X, _, (phi, bias) = _inputs(4096, 2048, synth.BF16, 5500)
    dX, dphi, dbias = to_device(X), to_device(phi), to_device(bias)
    with pytest.raises(RuntimeError):
        mhc.pre_ex(dX, dphi, dbias, mhc.PRE_ONE_PASS)
    _, _, used = mhc.pre_ex(dX, dphi, dbias, mhc.PRE_AUTO)
    torch.cuda.synchronize()
    assert used == mhc.PRE_TWO_PASS


@pytest.mark.parametrize("L", [0, 1, 7, 60])
def test_n8_amax_matches_oracle(mhc, oracle_lib, L):
    n, T = 8, 300
    m = n * n + 2 * n
    rng = np.random.default_rng(5600 + L)
    Hfull = np.zeros((L, T, m), np.float32)
    Hfull[:, :, n:n + n * n] = np.eye(n).reshape(1, 1, -1) + 0.2 * rng.standard_normal((L, T, n * n))
    r = mhc.amax(to_device(Hfull), n)
    torch.cuda.synchronize()
    ref = oracle_lib.amax(Hfull, n)
    for k in ("amax", "gain_fwd", "gain_bwd"):
        assert_close(to_host(r[k]), ref[k], 1e-4, 1e-6, what=f"amax {k}")
    scale = np.abs(ref["composite"]).max(axis=(1, 2), keepdims=True)
    err = np.abs(to_host(r["composite"]) - ref["composite"])
    assert np.all(err <= 1e-4 * scale + 1e-6), float((err / scale).max())
