"""mhc_pre at small T: the split-K form with one 16-token tile per workgroup.

When the persistent two-pass form would launch fewer than 128 workgroups
(ceil(T / 32) x ceil(d / 256) < 128), mhc_pre splits d into slices of 64
positions and gives every (slice, 16-token tile) pair a workgroup of its
own; the finishing pass sums the slices' records in a fixed order.  Each
case compares every token with the oracle; a second test checks that tokens
computed in a small-T call agree with the same tokens inside a call large
enough for the persistent form.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL, assert_close, dname, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


def small_form(T, d):
    return -(-T // 32) * -(-d // 256) < 128


CASES = [
    # (n, d, dtype, T)
    (4, 4096, synth.BF16, 1),
    (4, 4096, synth.BF16, 15),
    (4, 4096, synth.BF16, 16),
    (4, 4096, synth.BF16, 17),
    (4, 4096, synth.BF16, 224),     # the largest T of the small form at d = 4096
    (4, 2048, synth.BF16, 97),
    (4, 256, synth.FP32, 1),
    (4, 256, synth.FP32, 64),       # the fp32 small workload's shape
    (4, 264, synth.BF16, 33),       # ragged last slice
    (2, 520, synth.BF16, 40),
    (1, 128, synth.FP32, 5),
]


@pytest.mark.parametrize("n,d,dtype,T", CASES, ids=[f"n{c[0]}_d{c[1]}_{dname(c[2])}_T{c[3]}" for c in CASES])
@pytest.mark.parametrize("maps", ["mhc", "hc"])
def test_small_t_every_token(mhc, oracle_lib, n, d, dtype, T, maps):
    assert small_form(T, d)
    w = synth.Workload(f"small_{n}_{d}_{T}", T=T, n=n, d=d, dtype=dtype, seed=1200 + n + d + T)
    X = synth.make_state(w)
    phi, bias = synth.make_params(w)
    alpha = (0.6, 0.9, -0.7)
    code = mhc.MAPS_HC if maps == "hc" else mhc.MAPS_MHC
    h, H, used = mhc.pre_ex(to_device(X), to_device(phi), to_device(bias), mhc.PRE_AUTO, alpha=alpha, eps=w.eps,
                            t_max=w.t_max, maps=code)
    torch.cuda.synchronize()
    assert used == mhc.PRE_TWO_PASS
    dn = dname(dtype)
    if maps == "hc":
        ref = oracle_lib.pre_hc(X, phi, bias, alpha, eps=w.eps)
        rtol, atol = TOL[(dn, "maps")]
        atol = atol * max(1.0, 4.0 * max(abs(a) for a in alpha))
    else:
        ref = oracle_lib.pre(X, phi, bias, alpha, eps=w.eps, t_max=w.t_max)
        rtol, atol = TOL[(dn, "maps")]
    assert_close(to_host(H), ref["H"], rtol, atol, what=f"{w.name} {maps} H")
    assert_close(to_host(h), ref["h"], *TOL[(dn, "state")], what=f"{w.name} {maps} h")


@pytest.mark.parametrize("n,d,dtype", [(4, 4096, synth.BF16), (4, 256, synth.FP32)])
def test_small_t_agrees_with_persistent_form(mhc, n, d, dtype):
    """The first tokens of a large call (persistent form) against the same
    tokens on their own (small-T form): the same per-slice partials summed in
    a different grouping, so equal to rounding."""
    Tbig = 4096 if d <= 256 else 1024
    Tsmall = 40
    assert not small_form(Tbig, d) and small_form(Tsmall, d)
    w = synth.Workload(f"forms_{d}", T=Tbig, n=n, d=d, dtype=dtype, seed=1300 + d)
    X = synth.make_state(w)
    phi, bias = (to_device(a) for a in synth.make_params(w))
    dX = to_device(X)
    hb, Hb = mhc.pre(dX, phi, bias, alpha=(1.0, 1.0, 1.0), algo=mhc.PRE_TWO_PASS)
    hs, Hs = mhc.pre(dX[:Tsmall].contiguous(), phi, bias, alpha=(1.0, 1.0, 1.0), algo=mhc.PRE_TWO_PASS)
    torch.cuda.synchronize()
    assert float((Hb[:Tsmall] - Hs).abs().max()) < 1e-5
    dh = (hb[:Tsmall].float() - hs.float()).abs().max()
    assert float(dh) <= 1e-2 * float(hs.float().abs().max()) + 1e-6
