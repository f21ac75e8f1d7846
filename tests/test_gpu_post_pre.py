"""mhc_post_pre (layer l's mhc_post fused with layer l+1's mhc_pre) against
the separate entry points, bit for bit, and the 60-layer stack built on it
against the oracle."""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL, assert_close, check_stack_every_token, for_token_chunks, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


def _pair(mhc, w, inplace):
    """Layer 0's maps from mhc_pre, then layer 0's post + layer 1's pre both ways."""
    X = to_device(synth.make_state(w))
    Y = to_device(synth.make_sublayer_out(w))
    phi0, b0 = (to_device(a) for a in synth.make_params(w, layer=0))
    phi1, b1 = (to_device(a) for a in synth.make_params(synth.scaled(w, layers=2), layer=1))
    _, H0 = mhc.pre(X, phi0, b0, alpha=w.alpha, eps=w.eps, t_max=w.t_max)
    Xs = mhc.post(X, Y, H0)
    hs, Hs = mhc.pre(Xs, phi1, b1, alpha=w.alpha, eps=w.eps, t_max=w.t_max, algo=mhc.PRE_TWO_PASS)
    Xin = X.clone() if inplace else X
    Xf, hf, Hf = mhc.post_pre(Xin, Y, H0, phi1, b1, alpha=w.alpha, eps=w.eps, t_max=w.t_max,
                              out=Xin if inplace else None)
    torch.cuda.synchronize()
    return [to_host(a) for a in (Xs, hs, Hs, Xf, hf, Hf)]


CASES = [
    ("layer_bf16_T16384_d4096", {"T": 1100}),
    ("stack60_bf16_T4096_d2560", {"T": 300, "layers": 1, "sublayer": "given"}),     # ragged slice of d
    ("layer_fp32_T64_d256", {}),
    ("layer_bf16_T4096_d2048", {"T": 33}),
]


@pytest.mark.parametrize("name,changes", CASES, ids=[f"{c[0]}_T{c[1].get('T', 'all')}" for c in CASES])
@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
def test_post_pre_equals_separate_calls(mhc, name, changes, inplace):
    w = synth.scaled(synth.WORKLOADS[name], **changes)
    Xs, hs, Hs, Xf, hf, Hf = _pair(mhc, w, inplace)
    assert np.array_equal(Xs, Xf), "X_{l+1}"
    assert np.array_equal(hs, hf), "h_{l+1}"
    assert np.array_equal(Hs, Hf), "H_{l+1}"


@pytest.mark.parametrize("n", [1, 2])
def test_post_pre_fewer_streams(mhc, n):
    for dtype in (synth.BF16, synth.FP32):
        w = synth.Workload(f"post_pre_n{n}", T=150, n=n, d=520, dtype=dtype, seed=880 + n, alpha=(0.7, 0.9, -0.3))
        Xs, hs, Hs, Xf, hf, Hf = _pair(mhc, w, False)
        assert np.array_equal(Xs, Xf) and np.array_equal(hs, hf) and np.array_equal(Hs, Hf)


def _stack_fused(mhc, w, T, L, pingpong=False):
    """The L-layer stack as pre_0, then (0.5 GELU, post_pre) per layer, then a
    last post; in place, or with X_{l+1} in the other of two buffers (where
    MHC_PRE_AUTO may take the single pass)."""
    X0 = synth.make_state(w, T)
    phis, biases = zip(*(synth.make_params(w, layer=l) for l in range(L)))
    X = to_device(X0)
    other = torch.empty_like(X) if pingpong else X
    Hs = torch.empty((L, T, w.m), dtype=torch.float32, device="cuda")
    h, _ = mhc.pre(X, to_device(phis[0]), to_device(biases[0]), alpha=w.alpha, eps=w.eps, t_max=w.t_max, H=Hs[0])
    for l in range(L - 1):
        Y = mhc.gelu_half(h)
        Xn, h, _ = mhc.post_pre(X, Y, Hs[l], to_device(phis[l + 1]), to_device(biases[l + 1]), alpha=w.alpha,
                                eps=w.eps, t_max=w.t_max, out=other, H_next=Hs[l + 1])
        X, other = Xn, X
    X = mhc.post(X, mhc.gelu_half(h), Hs[L - 1], out=X)
    am = mhc.amax(Hs, w.n)
    torch.cuda.synchronize()
    return X0, np.stack(phis), np.stack(biases), to_host(X), to_host(Hs), {k: to_host(v) for k, v in am.items()}


@pytest.mark.parametrize("T,pingpong", [(40, False), (4096, False), (4096, True)])
def test_stack60_fused(mhc, oracle_lib, T, pingpong):
    """The 60-layer stack on mhc_post_pre: final state, every layer's maps and
    the per-token composite Amax against the oracle on every token (same
    criteria as the unfused stack).  In place the two-pass form runs; with two
    state buffers at T = 4096 MHC_PRE_AUTO takes the single pass (teams of 10
    at d = 2560, 10.7 tiles each)."""
    w = synth.WORKLOADS["stack60_bf16_T4096_d2560"]
    L = w.layers
    print(f"[post_pre] stack T={T} pingpong={pingpong}", flush=True)
    X0, phis, biases, Xg, Hg, am = _stack_fused(mhc, w, T, L, pingpong)
    check_stack_every_token(oracle_lib, w, X0, phis, biases, Xg, Hg, am, L)


# ---------------------------------------------------------------------------
# The single pass with layer l's post in front (MHC_PRE_ONE_PASS): X_{l+1} is
# formed in registers, stored, and used for layer l+1's projection and h
# without being read back.

ERR_FLIP = 0x5555555555555555


def _recomputed(ws) -> bool:
    hd = [int(v) & 0xFFFFFFFFFFFFFFFF for v in ws[:24].view(torch.int64).cpu()]
    return hd[0] == hd[2] ^ ERR_FLIP


def _inputs(w, alpha=None):
    X = synth.make_state(w)
    Y = synth.make_sublayer_out(w)
    phi0, b0 = synth.make_params(w, layer=0)
    phi1, b1 = synth.make_params(synth.scaled(w, layers=2), layer=1)
    return X, Y, phi0, b0, phi1, b1


def _one_pass_pair(mhc, w, algo, alpha=None):
    """Layer 0's maps, then (a) mhc_post + single-pass mhc_pre and (b)
    mhc_post_pre_ex(algo) on the same inputs."""
    alpha = w.alpha if alpha is None else alpha
    X, Y, phi0, b0, phi1, b1 = (to_device(a) for a in _inputs(w))
    _, H0 = mhc.pre(X, phi0, b0, alpha=alpha, eps=w.eps, t_max=w.t_max)
    Xs = mhc.post(X, Y, H0)
    ws1 = torch.zeros(mhc.pre_workspace_size(w.T, w.n, w.d, w.dtype), dtype=torch.uint8, device="cuda")
    hs, Hs, used_s = mhc.pre_ex(Xs, phi1, b1, mhc.PRE_ONE_PASS, alpha=alpha, eps=w.eps, t_max=w.t_max, workspace=ws1)
    ws2 = torch.zeros_like(ws1)
    Xf, hf, Hf, used_f = mhc.post_pre_ex(X, Y, H0, phi1, b1, algo, alpha=alpha, eps=w.eps, t_max=w.t_max,
                                         workspace=ws2)
    torch.cuda.synchronize()
    assert used_s == mhc.PRE_ONE_PASS and used_f == mhc.PRE_ONE_PASS
    assert not _recomputed(ws1)
    out = dict(X=to_host(X), Y=to_host(Y), H0=to_host(H0), Xs=to_host(Xs), hs=to_host(hs), Hs=to_host(Hs),
               Xf=to_host(Xf), hf=to_host(hf), Hf=to_host(Hf), fell_back=_recomputed(ws2))
    return out


ONE_PASS_CASES = [
    ("layer_bf16_T16384_d4096", {"T": 1024}),      # four tiles per team
    ("layer_bf16_T16384_d4096", {"T": 2048}),      # eight tiles per team: the exchange ring wraps
    ("layer_bf16_T16384_d4096", {"T": 4100}),      # ragged last tile, the ring wraps three times
    ("layer_bf16_T4096_d2048", {"T": 4096}),       # team of 8
    ("stack60_bf16_T4096_d2560", {"T": 1600, "layers": 1, "sublayer": "given"}),   # team of 10, ragged last tile
    ("layer_bf16_T16384_d4096", {"T": 2048, "d": 3000}),   # team of 12, the last slice ends inside a line
]


@pytest.mark.parametrize("name,changes", ONE_PASS_CASES,
                         ids=[f"{c[0]}_T{c[1]['T']}" + (f"_d{c[1]['d']}" if "d" in c[1] else "") for c in ONE_PASS_CASES])
def test_post_pre_one_pass_equals_separate_calls(mhc, name, changes):
    """Bit for bit the results of mhc_post followed by the single-pass mhc_pre."""
    w = synth.scaled(synth.WORKLOADS[name], **changes)
    print(f"[post_pre one pass] {w.name} T={w.T} d={w.d}", flush=True)
    r = _one_pass_pair(mhc, w, mhc.PRE_ONE_PASS, alpha=(1.0, 1.0, 1.0))
    assert not r["fell_back"], "an exchange wait ran out"
    assert np.array_equal(r["Xs"], r["Xf"]), "X_{l+1}"
    assert np.array_equal(r["hs"], r["hf"]), "h_{l+1}"
    assert np.array_equal(r["Hs"], r["Hf"]), "H_{l+1}"


@pytest.mark.parametrize("n", [1, 2])
def test_post_pre_one_pass_fewer_streams(mhc, n):
    w = synth.Workload(f"post_pre_one_pass_n{n}", T=1024, n=n, d=4096, dtype=synth.BF16, seed=990 + n,
                       alpha=(1.0, 0.5, -0.5))
    r = _one_pass_pair(mhc, w, mhc.PRE_ONE_PASS)
    assert not r["fell_back"]
    assert np.array_equal(r["Xs"], r["Xf"]) and np.array_equal(r["hs"], r["hf"]) and np.array_equal(r["Hs"], r["Hf"])


def test_post_pre_one_pass_fallback_is_bitwise(mhc):
    """The recomputing kernel (every workgroup starting broken) gives the
    single pass's bits."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=2100)
    a = _one_pass_pair(mhc, w, mhc.PRE_ONE_PASS)
    b = _one_pass_pair(mhc, w, mhc.PRE_ONE_PASS_FALLBACK_TEST)
    assert not a["fell_back"] and b["fell_back"]
    for k in ("Xf", "hf", "Hf"):
        assert np.array_equal(a[k], b[k]), k


def _oracle_every_token(o, w, r, alpha):
    """X_{l+1} against the oracle's post of (X, Y, H0), and layer l+1's h and
    H against the oracle's pre of the stored X_{l+1}, on every token."""
    phi1, b1 = synth.make_params(synth.scaled(w, layers=2), layer=1)

    def cmp(tok):
        xo = o.post(r["X"], r["Y"], r["H0"][tok], tokens=tok)
        assert_close(r["Xf"][tok], xo, *TOL[("bf16", "state")], what=f"X_(l+1), tokens {tok[0]}..")
        ref = o.pre(r["Xf"], phi1, b1, alpha, eps=w.eps, t_max=w.t_max, tokens=tok)
        assert_close(r["Hf"][tok], ref["H"], *TOL[("bf16", "maps")], what=f"H_(l+1), tokens {tok[0]}..")
        assert_close(r["hf"][tok], ref["h"], *TOL[("bf16", "state")], what=f"h_(l+1), tokens {tok[0]}..")

    for_token_chunks(cmp, w.T)


@pytest.mark.parametrize("T", [4096, 16384])
def test_post_pre_one_pass_every_token(mhc, oracle_lib, T):
    """The single pass with the post in front against the oracle on every
    token, at the headline shape (T = 16384: 64 tiles per team) and at a
    quarter of it."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=T)
    print(f"[post_pre one pass] oracle every token T={T}", flush=True)
    r = _one_pass_pair(mhc, w, mhc.PRE_ONE_PASS)
    assert not r["fell_back"]
    _oracle_every_token(oracle_lib, w, r, w.alpha)


def test_auto_takes_single_pass_for_teams_of_ten(mhc):
    """At d = 2560 a team has 10 members, so 2 of each XCD's 32 compute units
    stay idle; from 10 tiles per team (T = 4096) MHC_PRE_AUTO still takes the
    single pass for both entry points, bit for bit the forced form, and the
    two-pass form below that (T = 3072, 8 tiles per team)."""
    for T, want in ((4096, mhc.PRE_ONE_PASS), (3072, mhc.PRE_TWO_PASS)):
        w = synth.scaled(synth.WORKLOADS["stack60_bf16_T4096_d2560"], T=T, layers=1, sublayer="given")
        X, Y, phi0, b0, phi1, b1 = (to_device(a) for a in _inputs(w))
        kw = dict(alpha=w.alpha, eps=w.eps, t_max=w.t_max)
        ha, Ha, used = mhc.pre_ex(X, phi0, b0, mhc.PRE_AUTO, **kw)
        assert used == want, (T, used)
        hf, Hf, _ = mhc.pre_ex(X, phi0, b0, want, **kw)
        assert torch.equal(ha, hf) and torch.equal(Ha, Hf)
        auto = mhc.post_pre_ex(X, Y, Ha, phi1, b1, mhc.PRE_AUTO, **kw)
        assert auto[3] == want, (T, auto[3])
        forced = mhc.post_pre_ex(X, Y, Ha, phi1, b1, want, **kw)
        assert all(torch.equal(a, b) for a, b in zip(auto[:3], forced[:3]))
    torch.cuda.synchronize()


def test_post_pre_auto_and_alias(mhc):
    """AUTO takes the single pass (measured faster) when X_out is a buffer of
    its own and the two-pass form in place, each bit for bit the form it
    reports; the single pass refuses X_out == X."""
    w = synth.WORKLOADS["layer_bf16_T16384_d4096"]
    X, Y, phi0, b0, phi1, b1 = (to_device(a) for a in _inputs(w))
    _, H0 = mhc.pre(X, phi0, b0, alpha=w.alpha, eps=w.eps, t_max=w.t_max)
    auto = mhc.post_pre_ex(X, Y, H0, phi1, b1, mhc.PRE_AUTO, alpha=w.alpha)
    assert auto[3] == mhc.PRE_ONE_PASS
    one = mhc.post_pre_ex(X, Y, H0, phi1, b1, mhc.PRE_ONE_PASS, alpha=w.alpha)
    assert all(torch.equal(a, b) for a, b in zip(auto[:3], one[:3]))
    Xc = X.clone()
    inpl = mhc.post_pre_ex(Xc, Y, H0, phi1, b1, mhc.PRE_AUTO, alpha=w.alpha, out=Xc)
    assert inpl[3] == mhc.PRE_TWO_PASS
    two = mhc.post_pre_ex(X, Y, H0, phi1, b1, mhc.PRE_TWO_PASS, alpha=w.alpha)
    assert all(torch.equal(a, b) for a, b in zip(inpl[:3], two[:3]))
    assert torch.equal(auto[0], two[0])          # X_{l+1}: the same mix in both forms
    with pytest.raises(mhc.MhcError) as ei:
        mhc.post_pre_ex(X, Y, H0, phi1, b1, mhc.PRE_ONE_PASS, alpha=w.alpha, out=X)
    assert ei.value.status == 6
    torch.cuda.synchronize()
