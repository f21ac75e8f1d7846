"""Entry points captured into a HIP graph (torch.cuda.CUDAGraph).

mhc_pre's single pass takes its exchange tag from a sequence number in the
workspace header, which the kernel after it advances, so a replayed capture
gets a fresh tag every time.  Captured work is replayed several times with
eager calls on the same workspace and synchronisations in between; every
replay must give the eager results bit for bit.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ERR_FLIP = 0x5555555555555555


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


def _header(ws):
    return [int(v) & 0xFFFFFFFFFFFFFFFF for v in ws[:24].view(torch.int64).cpu()]


@pytest.mark.parametrize("algo", ["auto", "fallback_test"])
def test_forward_step_in_a_graph(mhc, algo):
    """The forward step (mhc_pre in the single pass, mhc_post, mhc_amax)
    captured once and replayed 4 times; with the testing aid every replay runs
    the single pass's fallback, which must give the same bits too."""
    T, n, d, m = 12288, 4, 4096, 24            # AUTO takes the single pass here
    g = torch.Generator(device="cuda").manual_seed(31)
    X = torch.randn(T, n, d, device="cuda", generator=g).to(torch.bfloat16)
    Y = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
    phi = torch.randn(n * d, m, device="cuda", generator=g) * 0.02
    bias = torch.randn(m, device="cuda", generator=g) * 0.1
    alpha = (1.0, 1.0, 1.0)
    ws = torch.zeros(mhc.pre_workspace_size(T, n, d, mhc.MHC_BF16), dtype=torch.uint8, device="cuda")
    h = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    H = torch.empty((T, m), device="cuda")
    Xo = torch.empty_like(X)
    amax = torch.empty(T, device="cuda")
    code = mhc.PRE_AUTO if algo == "auto" else mhc.PRE_ONE_PASS_FALLBACK_TEST

    h_ref, H_ref, used_eager = mhc.pre_ex(X, phi, bias, mhc.PRE_AUTO, alpha=alpha, workspace=ws)
    assert used_eager == mhc.PRE_ONE_PASS
    Xo_ref = mhc.post(X, Y, H_ref)
    a_ref = mhc.amax(H_ref.unsqueeze(0).contiguous(), n, want_all=False)["amax"]
    torch.cuda.synchronize()
    hd = _header(ws)
    assert hd[0] != hd[2] ^ ERR_FLIP
    refs = [t.clone() for t in (h_ref, H_ref, Xo_ref, a_ref)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    used = {}
    with torch.cuda.graph(graph, stream=s):
        _, _, used["captured"] = mhc.pre_ex(X, phi, bias, code, alpha=alpha, h=h, H=H, workspace=ws)
        mhc.post(X, Y, H, out=Xo)
        mhc.amax(H.unsqueeze(0), n, out_amax=amax, want_all=False)
    assert used["captured"] == mhc.PRE_ONE_PASS
    torch.cuda.synchronize()

    seq = _header(ws)[1]
    for r in range(4):
        for t in (h, H, Xo, amax):
            t.zero_()
        # eager work between replays: a single-pass call on the same workspace
        mhc.pre_ex(X, phi, bias, mhc.PRE_ONE_PASS, alpha=(0.5, 0.5, 0.5), workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        hd = _header(ws)
        assert hd[1] == seq + 2 * (r + 1), "every call, eager or replayed, advances the sequence number"
        assert (hd[0] == hd[2] ^ ERR_FLIP) == (algo != "auto"), f"replay {r}: unexpected fallback state"
        for got, want, name in zip((h, H, Xo, amax), refs, ("h", "H", "X'", "amax")):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager single-pass result"


def test_backward_and_post_pre_in_a_graph(mhc):
    """mhc_post_bwd_ex (tiled, with its workspace), mhc_pre_bwd and
    mhc_post_pre captured into one graph, replayed several times with eager
    work and synchronisations in between: every replay gives the eager
    results bit for bit (no entry point records a memset)."""
    T, n, d, m = 2048, 4, 2048, 24
    g = torch.Generator(device="cuda").manual_seed(37)
    X = torch.randn(T, n, d, device="cuda", generator=g).to(torch.bfloat16)
    Y = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
    G = torch.randn(T, n, d, device="cuda", generator=g).to(torch.bfloat16)
    D = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
    phi = torch.randn(n * d, m, device="cuda", generator=g) * 0.02
    bias = torch.randn(m, device="cuda", generator=g) * 0.1
    alpha = (0.7, 1.1, 0.4)
    _, H = mhc.pre(X, phi, bias, alpha=alpha)
    wsp = torch.empty(mhc.post_bwd_workspace_size(T, n, d, mhc.MHC_BF16), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(mhc.pre_bwd_workspace_size(T, n, d, mhc.MHC_BF16), dtype=torch.uint8, device="cuda")
    wsf = torch.empty(mhc.pre_workspace_size(T, n, d, mhc.MHC_BF16), dtype=torch.uint8, device="cuda")
    dX, dY = torch.empty_like(X), torch.empty_like(Y)
    dH = torch.zeros((T, m), device="cuda")
    dphi, dbias, dalpha = torch.empty((n * d, m), device="cuda"), torch.empty(m, device="cuda"), torch.empty(3, device="cuda")
    Xn, hn, Hn = torch.empty_like(X), torch.empty_like(Y), torch.empty((T, m), device="cuda")

    def run():
        mhc.post_bwd(X, Y, H, G, dX=dX, dY=dY, dH=dH, workspace=wsp)
        mhc.pre_bwd(X, phi, bias, D, dH, dX, alpha=alpha, dphi=dphi, dbias=dbias, dalpha=dalpha, workspace=wsb)
        mhc.post_pre(X, Y, H, phi, bias, alpha=alpha, out=Xn, h=hn, H_next=Hn, workspace=wsf)

    outs = (dX, dY, dH, dphi, dbias, dalpha, Xn, hn, Hn)
    run()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        run()
    for r in range(4):
        for t in outs:
            t.zero_()
        mhc.pre(X, phi, bias, alpha=(0.5, 0.5, 0.5), workspace=wsf)     # eager work on a shared workspace
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(outs, refs)):
            assert torch.equal(got, want), f"replay {r}: output {k} differs from the eager run"


def test_post_pre_single_pass_in_a_graph(mhc):
    """mhc_post_pre in its single pass (layer l's post in front of layer
    l+1's pre) captured and replayed 4 times with eager single-pass calls on
    the same workspace in between: every replay gives the eager bits."""
    T, n, d, m = 12288, 4, 4096, 24
    g = torch.Generator(device="cuda").manual_seed(41)
    X = torch.randn(T, n, d, device="cuda", generator=g).to(torch.bfloat16)
    Y = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
    phi = torch.randn(n * d, m, device="cuda", generator=g) * 0.02
    bias = torch.randn(m, device="cuda", generator=g) * 0.1
    alpha = (1.0, 1.0, 1.0)
    _, H = mhc.pre(X, phi, bias, alpha=alpha)
    ws = torch.zeros(mhc.pre_workspace_size(T, n, d, mhc.MHC_BF16), dtype=torch.uint8, device="cuda")
    Xn, hn, Hn = torch.empty_like(X), torch.empty_like(Y), torch.empty((T, m), device="cuda")
    Xr, hr, Hr, used = mhc.post_pre_ex(X, Y, H, phi, bias, mhc.PRE_ONE_PASS, alpha=alpha, workspace=ws)
    assert used == mhc.PRE_ONE_PASS
    torch.cuda.synchronize()
    hd = _header(ws)
    assert hd[0] != hd[2] ^ ERR_FLIP
    refs = [t.clone() for t in (Xr, hr, Hr)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        mhc.post_pre_ex(X, Y, H, phi, bias, mhc.PRE_ONE_PASS, alpha=alpha, out=Xn, h=hn, H_next=Hn, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        for t in (Xn, hn, Hn):
            t.zero_()
        mhc.post_pre_ex(X, Y, H, phi, bias, mhc.PRE_ONE_PASS, alpha=(0.5, 0.5, 0.5), workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        hd = _header(ws)
        assert hd[0] != hd[2] ^ ERR_FLIP, f"replay {r}: a wait ran out"
        for got, want, name in zip((Xn, hn, Hn), refs, ("X_(l+1)", "h", "H")):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager result"
