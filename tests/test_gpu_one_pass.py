"""The single-pass form of mhc_pre (MHC_PRE_ONE_PASS) against the oracle.

It applies to bf16 state with ceil(d / 256) in [8, 16] and at least one
16-token tile per team of workgroups; a team's members split d and exchange
per-token sums through their XCD's L2.  Each case checks that the one-pass
form really ran, that no internal wait ran out (the workspace header's error
word does not hold the call's tag), and that the results match the oracle
like the two-pass form's do.

The exchange ring holds 5 tiles per team, so a team that walks more than 5
tiles reuses its slots: T >= 1280 at d = 4096 (16 teams) and T >= 2560 at
d = 2048 (32 teams).  The cases below cover both sides of that line, and the
full-size workload (64 tiles per team) is compared on every token.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL, assert_close, for_token_chunks, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


ERR_FLIP = 0x5555555555555555
TAG_BIT = 1 << 63


def header(ws):
    """The workspace header's words (unsigned): error word, next sequence
    number, tag of the last one-pass call."""
    return [int(v) & 0xFFFFFFFFFFFFFFFF for v in ws[:24].view(torch.int64).cpu()]


def recomputed(ws) -> bool:
    """Whether the last one-pass call on ws was recomputed by its fallback kernel."""
    hd = header(ws)
    return hd[0] == hd[2] ^ ERR_FLIP


def _run(mhc, w, X, phi, bias, alpha, algo, maps=0):
    dX, dphi, dbias = to_device(X), to_device(phi), to_device(bias)
    ws = torch.zeros(mhc.pre_workspace_size(w.T, w.n, w.d, w.dtype), dtype=torch.uint8, device="cuda")
    h, H, used = mhc.pre_ex(dX, dphi, dbias, algo, alpha=alpha, eps=w.eps, t_max=w.t_max, workspace=ws, maps=maps)
    torch.cuda.synchronize()
    return to_host(h), to_host(H), used, recomputed(ws)


def _check(mhc, o, w, alpha=None):
    """Every token of the workload against the oracle (threaded over token chunks)."""
    alpha = w.alpha if alpha is None else alpha
    X = synth.make_state(w)
    phi, bias = synth.make_params(w)
    h, H, used, fell_back = _run(mhc, w, X, phi, bias, alpha, mhc.PRE_ONE_PASS)
    assert used == mhc.PRE_ONE_PASS
    assert not fell_back, "an exchange wait ran out"

    def cmp(tok):
        ref = o.pre(X, phi, bias, alpha, eps=w.eps, t_max=w.t_max, tokens=tok)
        assert_close(H[tok], ref["H"], *TOL[("bf16", "maps")], what=f"{w.name} one-pass H, tokens {tok[0]}..")
        assert_close(h[tok], ref["h"], *TOL[("bf16", "state")], what=f"{w.name} one-pass h, tokens {tok[0]}..")

    for_token_chunks(cmp, w.T)
    return X, phi, bias, h, H


CASES = [
    ("layer_bf16_T16384_d4096", {"T": 1024}),            # team of 16, exactly four tiles per team
    ("layer_bf16_T16384_d4096", {"T": 1100}),            # ragged last tile
    ("layer_bf16_T16384_d4096", {"T": 2048}),            # 8 tiles per team: the exchange ring wraps
    ("layer_bf16_T16384_d4096", {"T": 4100}),            # 16-17 tiles per team, ragged: wraps three times
    ("layer_bf16_T4096_d2048", {"T": 2048}),             # team of 8
    ("layer_bf16_T4096_d2048", {"T": 4096}),             # team of 8, 8 tiles per team: wraps
    ("stack60_bf16_T4096_d2560", {"T": 1600, "layers": 1, "sublayer": "given"}),   # team of 10, ragged last tile
    ("stack60_bf16_T4096_d2560", {"T": 4096, "layers": 1, "sublayer": "given"}),   # team of 10, ~11 tiles each
    # d not a multiple of 256: the last member's slice ends inside a line
    # (lanes of a 128-byte line partly past d), teams of 12 and 9
    ("layer_bf16_T16384_d4096", {"T": 2048, "d": 3000}),
    ("layer_bf16_T16384_d4096", {"T": 1500, "d": 2056}),
]


@pytest.mark.parametrize("name,changes", CASES,
                         ids=[f"{c[0]}_T{c[1]['T']}" + (f"_d{c[1]['d']}" if "d" in c[1] else "") for c in CASES])
@pytest.mark.parametrize("alpha", [None, (1.0, 1.0, 1.0)], ids=["alpha_cfg", "alpha_1"])
def test_one_pass_every_token(mhc, oracle_lib, name, changes, alpha):
    w = synth.scaled(synth.WORKLOADS[name], **changes)
    _check(mhc, oracle_lib, w, alpha=alpha)


def test_one_pass_twice_the_headline_size(mhc, oracle_lib):
    """T = 32768 (1 GiB of state, 128 tiles per team: the exchange ring
    wraps 25 times), every token against the oracle."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=32768)
    print(f"[one pass] every token at T={w.T}", flush=True)
    _check(mhc, oracle_lib, w)


@pytest.mark.parametrize("n", [1, 2])
def test_one_pass_fewer_streams(mhc, oracle_lib, n):
    w = synth.Workload(f"one_pass_n{n}", T=1024, n=n, d=4096, dtype=synth.BF16, seed=777 + n)
    _check(mhc, oracle_lib, w, alpha=(1.0, 0.5, -0.5))


@pytest.mark.slow
@pytest.mark.parametrize("alpha", [None, (1.0, 1.0, 1.0)], ids=["alpha_cfg", "alpha_1"])
def test_one_pass_full_size_every_token(mhc, oracle_lib, alpha):
    """The headline workload (T = 16384, d = 4096: 16 teams walking 64 tiles
    each, the exchange ring wrapping 12 times) on every token."""
    w = synth.WORKLOADS["layer_bf16_T16384_d4096"]
    print(f"[one-pass] full size, alpha {alpha}", flush=True)
    _check(mhc, oracle_lib, w, alpha=alpha)


def test_one_pass_deterministic_and_agrees_with_two_pass(mhc):
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=2048)
    X = synth.make_state(w)
    phi, bias = synth.make_params(w)
    a = _run(mhc, w, X, phi, bias, (1.0, 1.0, 1.0), mhc.PRE_ONE_PASS)
    b = _run(mhc, w, X, phi, bias, (1.0, 1.0, 1.0), mhc.PRE_ONE_PASS)
    c = _run(mhc, w, X, phi, bias, (1.0, 1.0, 1.0), mhc.PRE_TWO_PASS)
    assert a[2] == mhc.PRE_ONE_PASS and c[2] == mhc.PRE_TWO_PASS
    assert not a[3] and not b[3]
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
    h, H, used, fell_back = _run(mhc, w, X, phi, bias, alpha, mhc.PRE_ONE_PASS, maps=mhc.MAPS_HC)
    assert used == mhc.PRE_ONE_PASS and not fell_back
    rtol, atol = TOL[("bf16", "maps")]

    def cmp(tok):
        ref = oracle_lib.pre_hc(X, phi, bias, alpha, eps=w.eps, tokens=tok)
        assert_close(H[tok], ref["H"], rtol, atol * 4.0 * max(alpha), what=f"one-pass HC H, tokens {tok[0]}..")
        assert_close(h[tok], ref["h"], *TOL[("bf16", "state")], what=f"one-pass HC h, tokens {tok[0]}..")

    for_token_chunks(cmp, T)


@pytest.mark.parametrize("init", ["zeros", "garbage"])
def test_one_pass_repeated_calls_same_workspace(mhc, init):
    """Back-to-back calls on one workspace (the exchange ring keeps the last
    call's words): every call must produce the same bits, none may fall back,
    and each advances the header's sequence number by one.  The workspace
    starts zeroed, or filled with a byte pattern (any initial contents work)."""
    w = synth.scaled(synth.WORKLOADS["layer_bf16_T16384_d4096"], T=4096)
    X = to_device(synth.make_state(w))
    phi, bias = (to_device(a) for a in synth.make_params(w))
    nbytes = mhc.pre_workspace_size(w.T, w.n, w.d, w.dtype)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    if init == "garbage":
        ws.fill_(0x5A)
    outs = []
    seq0 = None
    for k in range(6):
        h, H, used = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=w.alpha, workspace=ws)
        assert used == mhc.PRE_ONE_PASS
        outs.append((to_host(h).copy(), to_host(H).copy()))
        hd = header(ws)
        assert not recomputed(ws), f"call {k} fell back"
        assert hd[2] == ((hd[1] - 1) % TAG_BIT) | TAG_BIT           # this call's tag: the sequence number before
        seq0 = hd[1] - k if seq0 is None else seq0
        assert hd[1] == seq0 + k                                    # one step per call
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
        h, H, used, fell_back = _run(mhc, w, X, phi, bias, alpha, algo)
        assert used == algo and not fell_back
        assert np.all(np.isfinite(H))
        assert_close(H, ref["H"], *TOL[("bf16", "maps")], what=f"large state H ({algo})")
        assert_close(h, ref["h"], *TOL[("bf16", "state")], what=f"large state h ({algo})")


@pytest.mark.parametrize("maps", ["mhc", "hc"])
@pytest.mark.parametrize("T,n", [(300, 4), (4100, 4), (1024, 2), (1024, 1)])
def test_one_pass_fallback(mhc, T, n, maps):
    """A single pass whose waits run out is recomputed by the kernel that
    follows it, with the single pass's own arithmetic: the results are the
    same bits as an undisturbed call.  The testing aid
    MHC_PRE_ONE_PASS_FALLBACK_TEST makes every workgroup start broken (the
    condition a team that is not all resident meets).  The header then holds
    the call's tag in its error word; the next ordinary call leaves that word
    alone and does not fall back."""
    w = synth.Workload(f"fallback_T{T}_n{n}", T=T, n=n, d=4096, dtype=synth.BF16, seed=7300 + T + n)
    code = mhc.MAPS_HC if maps == "hc" else mhc.MAPS_MHC
    X = to_device(synth.make_state(w))
    phi, bias = (to_device(a) for a in synth.make_params(w))
    alpha = (0.9, 1.1, 0.7)
    ws = torch.full((mhc.pre_workspace_size(w.T, w.n, w.d, w.dtype),), 0xA5, dtype=torch.uint8, device="cuda")
    h0, H0, used0 = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=alpha, workspace=ws, maps=code)
    assert used0 == mhc.PRE_ONE_PASS and not recomputed(ws)
    ref = (to_host(h0).copy(), to_host(H0).copy())
    h1, H1, used1 = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS_FALLBACK_TEST, alpha=alpha, workspace=ws, maps=code)
    torch.cuda.synchronize()
    hd = header(ws)
    assert used1 == mhc.PRE_ONE_PASS and recomputed(ws)
    assert np.array_equal(to_host(h1), ref[0]) and np.array_equal(to_host(H1), ref[1])
    h3, H3, used3 = mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=alpha, workspace=ws, maps=code)
    torch.cuda.synchronize()
    hd3 = header(ws)
    assert hd3[0] == hd[0] and not recomputed(ws)            # error word kept, this call did not fall back
    assert np.array_equal(to_host(h3), ref[0]) and np.array_equal(to_host(H3), ref[1])
    h2, H2, _ = mhc.pre_ex(X, phi, bias, mhc.PRE_TWO_PASS, alpha=alpha, maps=code)
    assert np.max(np.abs(to_host(H2).astype(np.float64) - ref[1])) < 1e-5
