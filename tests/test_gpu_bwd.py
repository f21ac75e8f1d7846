"""mhc_post_bwd + mhc_pre_bwd against the oracle's backward.

The checked quantity is the gradient of sum_t <G_t, X'_t> + <D_t, h_t> with
G = dX' and D = dh drawn as inputs (the sublayer stays outside the layer).
The chain is the one a training step runs: mhc_post_bwd writes dX (residual
part), dY and dH's res / post columns; mhc_pre_bwd adds the read map's and the
maps' share to dX and writes dphi, dbias, dalpha.  In the whole-dX form
mhc_post_bwd skips dX and mhc_pre_bwd_ex writes all of it from G.

Tolerances: dX and dY as the forward's state outputs (fp32: 1e-5 / 1e-6;
bf16: 2e-2 / 1e-2).  dH and the parameter gradients are fp32 sums over d or
over tokens: elementwise 1e-4 (dH) or 1e-3 (parameter gradients) relative
plus 1e-5 (dH) or 1e-4 (parameters) of the array's largest magnitude.  The
bound covers fp32 accumulation over up to 16384 terms and the fp32 Sinkhorn
backward (2 t_max steps of a division each, ~1e-6 relative); it is ~20x
tighter than a bf16 tolerance.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import synth
from gpu_helpers import TOL, assert_close, dname, to_device, to_host, values

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


def assert_scaled(got, ref, rtol, atol_frac, what):
    ref = np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    return assert_close(np.asarray(got, np.float64), ref, rtol, atol_frac * scale + 1e-30, what)


def _inputs(w, T=None):
    T = w.T if T is None else T
    X = synth.make_state(w, T)
    Y = synth.make_sublayer_out(w, T)
    G, D = synth.make_grads(w, T)
    phi, bias = synth.make_params(w)
    return X, Y, G, D, phi, bias


def _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, alpha, t_max=None, whole=False):
    """Forward maps, then the backward chain.  Returns host arrays.  whole:
    mhc_post_bwd skips dX, mhc_pre_bwd_ex writes all of it (into a buffer
    filled with NaN first, so a value it failed to write shows)."""
    t_max = w.t_max if t_max is None else t_max
    dX_, dY_, dG, dD = to_device(X), to_device(Y), to_device(G), to_device(D)
    dphi_, dbias_ = to_device(phi), to_device(bias)
    _, H = mhc.pre(dX_, dphi_, dbias_, alpha=alpha, eps=w.eps, t_max=t_max)
    m = w.m
    dH = torch.full((X.shape[0], m), 7.0, dtype=torch.float32, device="cuda")
    gX, gY, dH = mhc.post_bwd(dX_, dY_, H, dG, dH=dH, skip_dX=whole)
    torch.cuda.synchronize()
    if whole:
        assert gX is None
        gX = torch.full_like(dX_, float("nan"))
        dX_post = None
    else:
        dX_post = to_host(gX).copy()
    dH_host = to_host(dH).copy()
    gphi, gbias, galpha = mhc.pre_bwd(dX_, dphi_, dbias_, dD, dH, gX, alpha=alpha, eps=w.eps, t_max=t_max,
                                      G=dG if whole else None)
    torch.cuda.synchronize()
    return {"dX": to_host(gX), "dY": to_host(gY), "dH": dH_host, "dX_post": dX_post,
            "dphi": to_host(gphi), "dbias": to_host(gbias), "dalpha": to_host(galpha)}


def _check(o, w, got, X, Y, G, D, phi, bias, alpha, t_max=None, tokens=None, params=True):
    t_max = w.t_max if t_max is None else t_max
    n = w.n
    tok = np.arange(X.shape[0]) if tokens is None else tokens
    ref = o.bwd(X, Y, phi, bias, alpha, G, D, eps=w.eps, t_max=t_max, tokens=tok)
    dn = dname(w.dtype)
    assert np.all(got["dH"][:, :n] == 7.0), "mhc_post_bwd wrote the read map's columns of dH"
    assert_scaled(got["dH"][tok][:, n:], ref["dH"][:, n:], 1e-4, 1e-5, f"{w.name} dH")
    assert_close(got["dY"][tok], ref["dY"], *TOL[(dn, "state")], what=f"{w.name} dY")
    assert_close(got["dX"][tok], ref["dX"], *TOL[(dn, "state")], what=f"{w.name} dX")
    if params:
        assert_scaled(got["dbias"], ref["dbias"], 1e-3, 1e-4, f"{w.name} dbias")
        assert_scaled(got["dalpha"], ref["dalpha"], 1e-3, 1e-4, f"{w.name} dalpha")
        assert_scaled(got["dphi"], ref["dphi"], 1e-3, 1e-4, f"{w.name} dphi")
    return ref


CASES = [
    # (workload, changes, alpha)
    ("layer_fp32_T64_d256", {}, None),
    ("layer_fp32_T64_d256", {}, (1.0, 0.7, -0.4)),
    ("layer_fwdbwd_bf16_T16384_d4096", {"T": 1100}, None),          # ragged token tiles and chunks
    ("layer_fwdbwd_bf16_T16384_d4096", {"T": 257}, (1.0, 0.7, -0.4)),
    ("layer_bf16_T4096_d2048", {"T": 700}, None),
    ("stack60_bf16_T4096_d2560", {"T": 300, "layers": 1, "sublayer": "given"}, None),   # ragged slice of d
]


@pytest.mark.parametrize("name,changes,alpha", CASES,
                         ids=[f"{c[0]}_T{c[1].get('T', 'all')}_{'acfg' if c[2] is None else 'a1'}" for c in CASES])
@pytest.mark.parametrize("whole", [False, True], ids=["split_dX", "whole_dX"])
def test_backward_every_token(mhc, oracle_lib, name, changes, alpha, whole):
    w = synth.scaled(synth.WORKLOADS[name], **changes)
    alpha = w.alpha if alpha is None else alpha
    X, Y, G, D, phi, bias = _inputs(w)
    print(f"[bwd] {w.name} T={w.T} n={w.n} d={w.d} alpha={alpha} whole={whole}", flush=True)
    got = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, alpha, whole=whole)
    _check(oracle_lib, w, got, X, Y, G, D, phi, bias, alpha)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_whole_dx_matches_split_form(mhc, n):
    """The whole-dX form changes only dX (rounded once instead of twice): the
    other outputs are bit for bit those of the split form, and dX agrees to
    bf16 rounding."""
    w = synth.Workload(f"whole_dx_n{n}", T=700, n=n, d=1024, dtype=synth.BF16, seed=960 + n, alpha=(0.8, 1.1, -0.5))
    X, Y, G, D, phi, bias = _inputs(w)
    a = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, w.alpha)
    b = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, w.alpha, whole=True)
    for k in ("dY", "dH", "dphi", "dbias", "dalpha"):
        assert np.array_equal(a[k], b[k]), k
    assert np.all(np.isfinite(values(b["dX"])))
    assert_close(b["dX"], values(a["dX"]), 2e-2, 1e-2, "whole dX against split dX")


@pytest.mark.parametrize("n", [1, 2])
def test_backward_fewer_streams(mhc, oracle_lib, n):
    for dtype in (synth.FP32, synth.BF16):
        w = synth.Workload(f"bwd_n{n}_{dname(dtype)}", T=97, n=n, d=264, dtype=dtype, seed=900 + n)
        alpha = (0.9, 1.2, -0.7)
        X, Y, G, D, phi, bias = _inputs(w)
        for whole in (False, True):
            got = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, alpha, whole=whole)
            _check(oracle_lib, w, got, X, Y, G, D, phi, bias, alpha)


@pytest.mark.parametrize("t_max", [0, 1, 3])
def test_backward_few_sinkhorn_passes(mhc, oracle_lib, t_max):
    """Few Sinkhorn passes.  With none, H_res = exp(logits) is not normalised
    (entries near e^4 at a large alpha_res) and dX is a difference of terms
    ~100x larger than itself, beyond fp32's 1e-5; that case runs at the
    workload's alpha."""
    w = synth.Workload(f"bwd_tmax{t_max}", T=80, n=4, d=128, dtype=synth.FP32, seed=950 + t_max)
    alpha = (0.5, 1.5, 0.5) if t_max > 0 else w.alpha
    X, Y, G, D, phi, bias = _inputs(w)
    got = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, alpha, t_max=t_max)
    _check(oracle_lib, w, got, X, Y, G, D, phi, bias, alpha, t_max=t_max)


@pytest.mark.parametrize("t_max,dtype", [(21, synth.FP32), (40, synth.BF16)], ids=["tmax21_fp32", "tmax40_bf16"])
def test_backward_many_sinkhorn_passes(mhc, oracle_lib, t_max, dtype):
    """More Sinkhorn passes than the token kernel keeps in registers (20):
    its iterates then go to LDS, one wave per workgroup."""
    w = synth.Workload(f"bwd_tmax{t_max}", T=83, n=4, d=512, dtype=dtype, seed=960 + t_max)
    alpha = (0.5, 1.5, 0.5)
    X, Y, G, D, phi, bias = _inputs(w)
    for whole in (False, True):
        got = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, alpha, t_max=t_max, whole=whole)
        _check(oracle_lib, w, got, X, Y, G, D, phi, bias, alpha, t_max=t_max)


POST_FORMS = [
    # (T, n, d, dtype): d a multiple of 512 takes the tiled form when given a workspace
    (1, 4, 512, synth.BF16),
    (257, 4, 4096, synth.BF16),      # last 4-token tile holds one token
    (130, 4, 2560, synth.BF16),      # five slices
    (66, 2, 1024, synth.FP32),
    (33, 1, 1536, synth.BF16),
    (50, 4, 520, synth.BF16),        # not a multiple of 512: no workspace, scratch-free form only
]


@pytest.mark.parametrize("T,n,d,dtype", POST_FORMS, ids=[f"T{c[0]}_n{c[1]}_d{c[2]}_{dname(c[3])}" for c in POST_FORMS])
def test_post_bwd_forms(mhc, oracle_lib, T, n, d, dtype):
    """mhc_post_bwd (scratch-free) and mhc_post_bwd_ex (tiled, per-slice dot
    products added in slice order): dY and dH against the oracle, each form
    bitwise reproducible, dX and dY identical between the forms."""
    w = synth.Workload(f"postbwd_T{T}_n{n}_d{d}", T=T, n=n, d=d, dtype=dtype, seed=7000 + T + d)
    X, Y, G, D, phi, bias = _inputs(w)
    alpha = (0.8, 1.1, -0.6)
    dX_, dY_, dG = to_device(X), to_device(Y), to_device(G)
    _, H = mhc.pre(dX_, to_device(phi), to_device(bias), alpha=alpha, eps=w.eps, t_max=w.t_max)
    assert mhc.post_bwd_workspace_size(T, n, d, dtype) == (T * (d // 512) * (n * n + n) * 4 if d % 512 == 0 else 0)
    runs = {}
    for tiled in (False, True, True):
        dH = torch.full((T, w.m), 7.0, dtype=torch.float32, device="cuda")
        gX, gY, dH = mhc.post_bwd(dX_, dY_, H, dG, dH=dH, tiled=tiled)
        torch.cuda.synchronize()
        out = (to_host(gX).copy(), to_host(gY).copy(), to_host(dH).copy())
        if tiled in runs:
            for a, b in zip(out, runs[tiled]):
                assert np.array_equal(a, b), "tiled form not reproducible"
        runs[tiled] = out
    ref = oracle_lib.bwd(X, Y, phi, bias, alpha, G, D, eps=w.eps, t_max=w.t_max)
    dn = dname(dtype)
    for tiled, (gX, gY, dH) in runs.items():
        assert np.all(dH[:, :n] == 7.0), "mhc_post_bwd wrote the read map's columns of dH"
        assert_close(gY, ref["dY"], *TOL[(dn, "state")], what=f"{w.name} tiled={tiled} dY")
        assert_scaled(dH[:, n:], ref["dH"][:, n:], 1e-4, 1e-5, f"{w.name} tiled={tiled} dH")
    # dX (checked through the whole chain elsewhere) and dY: the same arithmetic per element in both forms
    assert np.array_equal(runs[False][0], runs[True][0]) and np.array_equal(runs[False][1], runs[True][1])
    if d % 512 != 0:
        # a workspace passed where the tiled form does not apply is not used: the scratch-free results
        dH = torch.full((T, w.m), 7.0, dtype=torch.float32, device="cuda")
        gX, gY, dH = mhc.post_bwd(dX_, dY_, H, dG, dH=dH, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        for a, b in zip((to_host(gX), to_host(gY), to_host(dH)), runs[False]):
            assert np.array_equal(a, b)


def test_backward_empty_and_deterministic(mhc):
    w = synth.scaled(synth.WORKLOADS["layer_fwdbwd_bf16_T16384_d4096"], T=512)
    X, Y, G, D, phi, bias = _inputs(w)
    a = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, w.alpha)
    b = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, w.alpha)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    # T = 0: parameter gradients are written as zeros.
    e = synth.scaled(w, T=0)
    X0 = to_device(np.zeros((0, w.n, w.d), np.uint16))
    D0 = to_device(np.zeros((0, w.d), np.uint16))
    dH0 = torch.zeros((0, w.m), dtype=torch.float32, device="cuda")
    dphi = torch.full((w.K, w.m), 3.0, device="cuda")
    dbias = torch.full((w.m,), 3.0, device="cuda")
    dalpha = torch.full((3,), 3.0, device="cuda")
    mhc.pre_bwd(X0, to_device(phi), to_device(bias), D0, dH0, X0.clone(), alpha=e.alpha, dphi=dphi, dbias=dbias,
                dalpha=dalpha)
    torch.cuda.synchronize()
    assert float(dphi.abs().max()) == 0.0 and float(dbias.abs().max()) == 0.0 and float(dalpha.abs().max()) == 0.0


@pytest.mark.slow
@pytest.mark.parametrize("whole", [False, True], ids=["split_dX", "whole_dX"])
def test_backward_full_size(mhc, oracle_lib, whole):
    """T = 16384, n = 4, d = 4096 bf16 in the launch configuration the
    benchmark times, checked on EVERY token: the oracle runs over 256-token
    chunks on host threads (each chunk's per-token gradients are compared as
    they come), and the parameter gradients are the chunks' sums added in
    chunk order."""
    w = synth.WORKLOADS["layer_fwdbwd_bf16_T16384_d4096"]
    X, Y, G, D, phi, bias = _inputs(w)
    print(f"[bwd] full size {w.name} whole={whole}", flush=True)
    got = _gpu_bwd(mhc, w, X, Y, G, D, phi, bias, w.alpha, whole=whole)
    n, T, chunk = w.n, w.T, 256
    assert np.all(got["dH"][:, :n] == 7.0), "mhc_post_bwd wrote the read map's columns of dH"
    dn = dname(w.dtype)
    dH_ref = np.empty((T, w.m))

    def run(s):
        tok = np.arange(s, min(T, s + chunk), dtype=np.int64)
        r = oracle_lib.bwd(X, Y, phi, bias, w.alpha, G, D, eps=w.eps, t_max=w.t_max, tokens=tok)
        assert_close(got["dY"][tok], r["dY"], *TOL[(dn, "state")], what=f"dY, tokens {s}..")
        assert_close(got["dX"][tok], r["dX"], *TOL[(dn, "state")], what=f"dX, tokens {s}..")
        dH_ref[tok] = r["dH"]
        return r["dphi"], r["dbias"], r["dalpha"]

    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(run, range(0, T, chunk)))
    assert_scaled(got["dH"][:, n:], dH_ref[:, n:], 1e-4, 1e-5, "full dH")
    dphi = np.zeros_like(parts[0][0])
    dbias = np.zeros_like(parts[0][1])
    dalpha = np.zeros_like(parts[0][2])
    for p in parts:
        dphi += p[0]
        dbias += p[1]
        dalpha += p[2]
    assert_scaled(got["dbias"], dbias, 1e-3, 1e-4, "full dbias")
    assert_scaled(got["dalpha"], dalpha, 1e-3, 1e-4, "full dalpha")
    assert_scaled(got["dphi"], dphi, 1e-3, 1e-4, "full dphi")
