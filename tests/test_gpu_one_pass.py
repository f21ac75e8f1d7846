"""The single-pass form of mhc_pre (MHC_PRE_ONE_PASS) against the oracle.

It applies to bf16 state with ceil(d / 256) in [8, 16] and at least one
16-token tile per team of workgroups; a team's members split d and exchange
per-token sums through their XCD's L2.  Each case checks that the one-pass
form really ran, that no internal wait ran out (the workspace's error word is
0), and that the results match the oracle like the two-pass form's do.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL, assert_close, sample_tokens, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


def _run(mhc, w, X, phi, bias, alpha, algo, maps=0):
    dX, dphi, dbias = to_device(X), to_device(phi), to_device(bias)
    ws = torch.zeros(mhc.pre_workspace_size(w.T, w.n, w.d, w.dtype), dtype=torch.uint8, device="cuda")
    h, H, used = mhc.pre_ex(dX, dphi, dbias, algo, alpha=alpha, eps=w.eps, t_max=w.t_max, workspace=ws, maps=maps)
    torch.cuda.synchronize()
    err_word = int(ws[:4].view(torch.int32).item())
    return to_host(h), to_host(H), used, err_word


def _check(mhc, o, w, alpha=None, tokens=None):
    alpha = w.alpha if alpha is None else alpha
    X = synth.make_state(w)
    phi, bias = synth.make_params(w)
    h, H, used, err = _run(mhc, w, X, phi, bias, alpha, mhc.PRE_ONE_PASS)
    assert used == mhc.PRE_ONE_PASS
    assert err == 0, "an exchange wait ran out"
    tok = np.arange(w.T, dtype=np.int64) if tokens is None else tokens
    ref = o.pre(X, phi, bias, alpha, eps=w.eps, t_max=w.t_max, tokens=tok)
    assert_close(H[tok], ref["H"], *TOL[("bf16", "maps")], what=f"{w.name} one-pass H")
    assert_close(h[tok], ref["h"], *TOL[("bf16", "state")], what=f"{w.name} one-pass h")
    return X, phi, bias, h, H


CASES = [
    ("layer_bf16_T16384_d4096", {"T": 1024}),            # team of 16, exactly two tiles per team
    ("layer_bf16_T16384_d4096", {"T": 1100}),            # ragged last tile
    ("layer_bf16_T4096_d2048", {"T": 2048}),             # team of 8
    ("stack60_bf16_T4096_d2560", {"T": 1600, "layers": 1, "sublayer": "given"}),   # team of 10, ragged slice
]


@pytest.mark.parametrize("name,changes", CASES, ids=[f"{c[0]}_T{c[1]['T']}" for c in CASES])
@pytest.mark.parametrize("alpha", [None, (1.0, 1.0, 1.0)], ids=["alpha_cfg", "alpha_1"])
def test_one_pass_every_token(mhc, oracle_lib, name, changes, alpha):
    w = synth.scaled(synth.WORKLOADS[name], **changes)
    _check(mhc, oracle_lib, w, alpha=alpha)


@pytest.mark.parametrize("n", [1, 2])
def test_one_pass_fewer_streams(mhc, oracle_lib, n):
    w = synth.Workload(f"one_pass_n{n}", T=1024, n=n, d=4096, dtype=synth.BF16, seed=777 + n)
    _check(mhc, oracle_lib, w, alpha=(1.0, 0.5, -0.5))


@pytest.mark.slow
def test_one_pass_full_size_sampled(mhc, oracle_lib):
    w = synth.WORKLOADS["layer_bf16_T16384_d4096"]
    _check(mhc, oracle_lib, w, tokens=sample_tokens(w.T, 64, tile=32))


def test_one_pass_deterministic_and_agrees_with_two_pass(mhc):
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=2048)
    X = synth.make_state(w)
    phi, bias = synth.make_params(w)
    a = _run(mhc, w, X, phi, bias, (1.0, 1.0, 1.0), mhc.PRE_ONE_PASS)
    b = _run(mhc, w, X, phi, bias, (1.0, 1.0, 1.0), mhc.PRE_ONE_PASS)
    c = _run(mhc, w, X, phi, bias, (1.0, 1.0, 1.0), mhc.PRE_TWO_PASS)
    assert a[2] == mhc.PRE_ONE_PASS and c[2] == mhc.PRE_TWO_PASS
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.max(np.abs(a[1].astype(np.float64) - c[1])) < 1e-5


def test_one_pass_refuses_what_it_does_not_cover(mhc):
    cases = [
        synth.Workload("fp32", T=2048, n=4, d=4096, dtype=synth.FP32),          # fp32 state
        synth.Workload("small_T", T=64, n=4, d=4096, dtype=synth.BF16),         # too few tiles
        synth.Workload("narrow", T=4096, n=4, d=1024, dtype=synth.BF16),        # team of 4
    ]
    for w in cases:
        X = to_device(synth.make_state(w))
        phi, bias = (to_device(a) for a in synth.make_params(w))
        with pytest.raises(mhc.MhcError) as ei:
            mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS)
        assert ei.value.status == 5
        h, H, used = mhc.pre_ex(X, phi, bias, mhc.PRE_AUTO)      # auto falls back
        assert used == mhc.PRE_TWO_PASS


@pytest.mark.parametrize("T", [1100, 16384])
def test_one_pass_hc_maps(mhc, oracle_lib, T):
    """The unconstrained HC maps through the single pass: same tolerance rule
    as the two-pass HC test (the absolute part scales with |alpha|)."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=T)
    X = synth.make_state(w)
    phi, bias = synth.make_params(w)
    alpha = (0.8, 0.6, 1.2)
    h, H, used, err = _run(mhc, w, X, phi, bias, alpha, mhc.PRE_ONE_PASS, maps=mhc.MAPS_HC)
    assert used == mhc.PRE_ONE_PASS and err == 0
    tok = np.arange(T, dtype=np.int64) if T < 2000 else sample_tokens(T, 48, tile=16)
    ref = oracle_lib.pre_hc(X, phi, bias, alpha, eps=w.eps, tokens=tok)
    rtol, atol = TOL[("bf16", "maps")]
    assert_close(H[tok], ref["H"], rtol, atol * 4.0 * max(alpha), what="one-pass HC H")
    assert_close(h[tok], ref["h"], *TOL[("bf16", "state")], what="one-pass HC h")


def test_one_pass_repeated_calls_same_workspace(mhc):
    """Back-to-back calls on one workspace (the exchange ring keeps the last
    call's words): every call must produce the same bits and a clear error word."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=4096)
    X = to_device(synth.make_state(w))
    phi, bias = (to_device(a) for a in synth.make_params(w))
    ws = torch.zeros(mhc.pre_workspace_size(w.T, w.n, w.d, w.dtype), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(6):
        h, H, used = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=w.alpha, workspace=ws)
        assert used == mhc.PRE_ONE_PASS
        outs.append((to_host(h).copy(), to_host(H).copy()))
    torch.cuda.synchronize()
    assert int(ws[:8].view(torch.int64).item()) == 0
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])


def test_large_state_sum_of_squares(mhc, oracle_lib):
    """Tokens scaled by 2^64 (|x| ~ 1e19, exact in bf16): their squares
    overflow fp32, so the single pass's fp32 sum of squares must fall back to
    fp64 like the two-pass form; every token still matches the oracle."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=1024)
    X = synth.make_state(w)
    f = synth.bf16_bits_to_f32(X)
    big = [3, 100, 517, 1023]
    f[big] *= np.float32(2.0 ** 64)
    f[200] *= np.float32(2.0 ** -64)
    X = (f.view(np.uint32) >> 16).astype(np.uint16)
    phi, bias = synth.make_params(w)
    alpha = (1.0, 1.0, 1.0)
    ref = oracle_lib.pre(X, phi, bias, alpha, eps=w.eps, t_max=w.t_max)
    for algo in (mhc.PRE_ONE_PASS, mhc.PRE_TWO_PASS):
        h, H, used, err = _run(mhc, w, X, phi, bias, alpha, algo)
        assert used == algo
        assert err == 0 or algo == mhc.PRE_TWO_PASS      # the two-pass form keeps records there
        assert np.all(np.isfinite(H))
        assert_close(H, ref["H"], *TOL[("bf16", "maps")], what=f"large state H ({algo})")
        assert_close(h, ref["h"], *TOL[("bf16", "state")], what=f"large state h ({algo})")


@pytest.mark.parametrize("maps", ["mhc", "hc"])
@pytest.mark.parametrize("T,n", [(300, 4), (4100, 4), (1024, 2), (1024, 1)])
def test_one_pass_fallback(mhc, monkeypatch, T, n, maps):
    """A single pass whose waits run out is recomputed by the gated two-pass
    launches that follow it.  The library's testing switch makes every
    workgroup start broken (the condition a team that is not all resident
    meets): the call must still return the two-pass form's results bit for
    bit, leave a non-zero sequence number in the error word, and the next
    call without the switch must leave that word alone and give the same
    results."""
    w = synth.Workload(f"fallback_T{T}_n{n}", T=T, n=n, d=4096, dtype=synth.BF16, seed=7300 + T + n)
    code = mhc.MAPS_HC if maps == "hc" else mhc.MAPS_MHC
    X = to_device(synth.make_state(w))
    phi, bias = (to_device(a) for a in synth.make_params(w))
    alpha = (0.9, 1.1, 0.7)
    ws = torch.full((mhc.pre_workspace_size(w.T, w.n, w.d, w.dtype),), 0xA5, dtype=torch.uint8, device="cuda")
    ws[:8].zero_()
    h2, H2, used2 = mhc.pre_ex(X, phi, bias, mhc.PRE_TWO_PASS, alpha=alpha, maps=code)
    ref = (to_host(h2).copy(), to_host(H2).copy())
    monkeypatch.setenv("MHC_TEST_ONE_PASS_FALLBACK", "1")
    h1, H1, used1 = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=alpha, workspace=ws, maps=code)
    torch.cuda.synchronize()
    err = int(ws[:8].view(torch.int64).item())
    assert used1 == mhc.PRE_ONE_PASS and err != 0
    assert np.array_equal(to_host(h1), ref[0]) and np.array_equal(to_host(H1), ref[1])
    monkeypatch.delenv("MHC_TEST_ONE_PASS_FALLBACK")
    h3, H3, used3 = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=alpha, workspace=ws, maps=code)
    torch.cuda.synchronize()
    assert int(ws[:8].view(torch.int64).item()) == err          # never cleared by the library
    h4, H4, _ = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=alpha, maps=code)
    assert np.array_equal(to_host(h3), to_host(h4)) and np.array_equal(to_host(H3), to_host(H4))
    assert np.max(np.abs(to_host(H3).astype(np.float64) - ref[1])) < 1e-5
