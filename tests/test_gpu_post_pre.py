"""mhc_post_pre (layer l's mhc_post fused with layer l+1's mhc_pre) against
the separate entry points, bit for bit, and the 60-layer stack built on it
against the oracle."""
import numpy as np
import pytest

import synth
from gpu_helpers import assert_close, check_stack_every_token, to_device, to_host

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


def _stack_fused(mhc, w, T, L):
    """The L-layer stack as pre_0, then (0.5 GELU, post_pre) per layer, then a last post."""
    X0 = synth.make_state(w, T)
    phis, biases = zip(*(synth.make_params(w, layer=l) for l in range(L)))
    X = to_device(X0)
    Hs = torch.empty((L, T, w.m), dtype=torch.float32, device="cuda")
    h, _ = mhc.pre(X, to_device(phis[0]), to_device(biases[0]), alpha=w.alpha, eps=w.eps, t_max=w.t_max, H=Hs[0])
    for l in range(L - 1):
        Y = mhc.gelu_half(h)
        X, h, _ = mhc.post_pre(X, Y, Hs[l], to_device(phis[l + 1]), to_device(biases[l + 1]), alpha=w.alpha,
                               eps=w.eps, t_max=w.t_max, out=X, H_next=Hs[l + 1])
    X = mhc.post(X, mhc.gelu_half(h), Hs[L - 1], out=X)
    am = mhc.amax(Hs, w.n)
    torch.cuda.synchronize()
    return X0, np.stack(phis), np.stack(biases), to_host(X), to_host(Hs), {k: to_host(v) for k, v in am.items()}


@pytest.mark.parametrize("T", [40, 4096])
def test_stack60_fused(mhc, oracle_lib, T):
    """The 60-layer stack on mhc_post_pre: final state, every layer's maps and
    the per-token composite Amax against the oracle on every token (same
    criteria as the unfused stack)."""
    w = synth.WORKLOADS["stack60_bf16_T4096_d2560"]
    L = w.layers
    print(f"[post_pre] stack T={T}", flush=True)
    X0, phis, biases, Xg, Hg, am = _stack_fused(mhc, w, T, L)
    check_stack_every_token(oracle_lib, w, X0, phis, biases, Xg, Hg, am, L)
