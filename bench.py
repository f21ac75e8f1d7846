"""Benchmark of the mHC layer forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: mhc_pre (RMSNorm, projection, gates, Sinkhorn,
aggregation) -> the given sublayer output Y -> mhc_post (mixing +
broadcast-add) -> mhc_amax over the layer's maps.  Default workload: T = 16384
tokens (batch 4 x seq 4096), n = 4 streams, d = 4096, bf16 state.

Prints ONE JSON line (stdout) with tokens/s, the achieved HBM bandwidth on
algorithmic bytes, the roofline of the dominant entry point (timed live with
HIP events on the stream the kernels run on) and the CPU oracle's rate on a
bounded sample.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, vendor figure
METRIC = "mHC fwd tokens/sec + achieved HBM GB/s (n=4, d=4096, bf16, 1 GPU)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(T, n, d, sbytes):
    """Bytes each entry point must move per call: one pass over its tensors,
    phi read once.  pre: X in, h and H out, phi; post: X, Y, the 20 mixing /
    write values per token in, X' out; amax (one layer): H_res in, amax out."""
    m = n * n + 2 * n
    pre = T * (n * d * sbytes + d * sbytes + 4 * m) + n * d * m * 4 + 4 * m
    post = T * (n * d * sbytes + d * sbytes + 4 * (n * n + n) + n * d * sbytes)
    amax = T * (4 * n * n + 4)
    return {"mhc_pre": pre, "mhc_post": post, "mhc_amax": amax}


def backward_min_bytes(T, n, d, sbytes):
    """The least the layer's backward can move: read X, G, Y and D once
    ((2n + 2) d values per token), write dX and dY once ((n + 1) d), plus one
    more pass over X for the parameter gradients (their per-token factors
    are known only after a full pass over the token): (4n + 3) d values per
    token, 155,648 B at n = 4, d = 4096, bf16."""
    return T * (4 * n + 3) * d * sbytes


def backward_bytes(T, n, d, sbytes):
    """Bytes the backward entry points move by design (split where the
    sublayer sits).  post_bwd: X, G, Y and the mixing / write maps in; dX, dY
    and their dH columns out.  pre_bwd recomputes the maps, so it reads X and
    D twice (the token's dlogits are known only after a full pass), dX once to
    update it and dH's columns; it writes dX, and reads phi and writes dphi
    once."""
    m = n * n + 2 * n
    K = n * d
    post = T * (3 * K * sbytes + 2 * d * sbytes + 8 * (n * n + n))
    pre = T * (3 * K * sbytes + 2 * d * sbytes + 4 * (n * n + n) + K * sbytes) + 2 * K * m * 4 + 4 * (m + 3)
    return {"mhc_post_bwd": post, "mhc_pre_bwd": pre}


def time_backward(mhc, torch, w, X, Y, phi, bias, H, steps, warmup, stream):
    """Average time of mhc_post_bwd and mhc_pre_bwd on the layer forward +
    backward workload's gradients (same shapes as the forward workload)."""
    import numpy as np

    import synth
    wb = synth.WORKLOADS["layer_fwdbwd_bf16_T16384_d4096"]
    if (wb.T, wb.n, wb.d, wb.dtype) != (w.T, w.n, w.d, w.dtype):
        return None

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)

    G, D = (dev(a) for a in synth.make_grads(wb))
    T, n, d = w.T, w.n, w.d
    m = n * n + 2 * n
    dX = torch.empty_like(X)
    dY = torch.empty_like(Y)
    dH = torch.zeros((T, m), dtype=torch.float32, device="cuda")
    dphi = torch.empty((n * d, m), dtype=torch.float32, device="cuda")
    dbias = torch.empty(m, dtype=torch.float32, device="cuda")
    dalpha = torch.empty(3, dtype=torch.float32, device="cuda")
    ws = torch.empty(mhc.pre_bwd_workspace_size(T, n, d, w.dtype), dtype=torch.uint8, device="cuda")
    ws_post = torch.empty(max(16, mhc.post_bwd_workspace_size(T, n, d, w.dtype)), dtype=torch.uint8, device="cuda")

    def post_split():
        mhc.post_bwd(X, Y, H, G, dX=dX, dY=dY, dH=dH, workspace=ws_post, stream=stream)

    def pre_split():
        mhc.pre_bwd(X, phi, bias, D, dH, dX, alpha=w.alpha, eps=w.eps, t_max=w.t_max, dphi=dphi, dbias=dbias,
                    dalpha=dalpha, workspace=ws, stream=stream)

    # The whole-dX pair: mhc_post_bwd skips dX, mhc_pre_bwd_ex writes all of it from G.
    def post_whole():
        mhc.post_bwd(X, Y, H, G, dY=dY, dH=dH, workspace=ws_post, stream=stream, skip_dX=True)

    def pre_whole():
        mhc.pre_bwd(X, phi, bias, D, dH, dX, alpha=w.alpha, eps=w.eps, t_max=w.t_max, dphi=dphi, dbias=dbias,
                    dalpha=dalpha, workspace=ws, stream=stream, G=G)

    def timed(calls, reps):
        """Average time of one round of `calls`, `reps` rounds back to back, events at the ends."""
        for _ in range(warmup):
            for c in calls:
                c()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            for c in calls:
                c()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps * 1e3

    sb = 2 if w.dtype == synth.BF16 else 4
    algo = backward_bytes(T, n, d, sb)
    least = backward_min_bytes(T, n, d, sb)
    out = {"workload": wb.name, "steps": steps,
           "timing": "each figure: `steps` rounds back to back, HIP events at the ends; total_us: the pair together"}
    for name, fn in (("mhc_post_bwd", post_split), ("mhc_pre_bwd", pre_split)):
        us = timed([fn], steps)
        out[name] = {"avg_us": us, "design_bytes": algo[name], "GBps_design_bytes": algo[name] / (us * 1e-6) / 1e9}
    tot_us = timed([post_split, pre_split], steps)
    out["total_us"] = tot_us
    out["min_bytes"] = least
    out["GBps"] = least / (tot_us * 1e-6) / 1e9
    out["frac_of_peak"] = out["GBps"] / HBM_PEAK_GBPS
    out["bytes_note"] = ("GBps and frac_of_peak use the least bytes the backward must move, (4n + 3) d values "
                         "per token (X, G, Y, D read once, dX and dY written once, one more pass over X); "
                         "GBps_design_bytes per entry point counts what each call moves by design")
    whole = {"mhc_post_bwd_without_dX_us": timed([post_whole], steps),
             "mhc_pre_bwd_ex_us": timed([pre_whole], steps)}
    whole["total_us"] = timed([post_whole, pre_whole], steps)
    whole["GBps"] = least / (whole["total_us"] * 1e-6) / 1e9
    whole["frac_of_peak"] = whole["GBps"] / HBM_PEAK_GBPS
    whole["note"] = ("mhc_post_bwd with dX NULL, then mhc_pre_bwd_ex with G: dX written once (X, G, Y read and dY "
                     "written by the first; X, D read twice, G read, dX written by the second)")
    out["whole_dX"] = whole
    # The scratch-free form of mhc_post_bwd (no workspace), for reference.
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    mhc.post_bwd(X, Y, H, G, dX=dX, dY=dY, dH=dH, tiled=False, stream=stream)
    sev[0].record(stream)
    for _ in range(steps):
        mhc.post_bwd(X, Y, H, G, dX=dX, dY=dY, dH=dH, tiled=False, stream=stream)
    sev[1].record(stream)
    torch.cuda.synchronize()
    out["mhc_post_bwd_scratch_free_us"] = sev[0].elapsed_time(sev[1]) / steps * 1e3
    out["fwd_bwd_tokens_per_s"] = None
    return out


def time_stack(mhc, torch, reps=5, warmup=2):
    """The 60-layer stack workload (T=4096, n=4, d=2560, F = 0.5 GELU): the
    whole stack timed with the separate entry points per layer (pre, F,
    post) and with mhc_post_pre chaining each layer's post into the next
    layer's pre; plus the per-token composite Amax over its maps.  X_{l+1}
    goes to the other of two state buffers (a training step keeps X_l for
    its backward anyway), which lets MHC_PRE_AUTO take the single pass."""
    import numpy as np

    import synth
    w = synth.WORKLOADS["stack60_bf16_T4096_d2560"]
    T, n, d, L, m = w.T, w.n, w.d, w.layers, w.m

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    X0 = dev(synth.make_state(w))
    params = [tuple(dev(a) for a in synth.make_params(w, layer=l)) for l in range(L)]
    XA, XB = torch.empty_like(X0), torch.empty_like(X0)
    h = torch.empty((T, d), dtype=X0.dtype, device="cuda")
    Y = torch.empty_like(h)
    Hs = torch.empty((L, T, m), dtype=torch.float32, device="cuda")
    ws = torch.empty(mhc.pre_workspace_size(T, n, d, w.dtype), dtype=torch.uint8, device="cuda")
    amax = torch.empty(T, dtype=torch.float32, device="cuda")
    kw = dict(alpha=w.alpha, eps=w.eps, t_max=w.t_max)

    def separate():
        XA.copy_(X0)
        X, Xn = XA, XB
        for l in range(L):
            mhc.pre(X, params[l][0], params[l][1], h=h, H=Hs[l], workspace=ws, **kw)
            mhc.gelu_half(h, out=Y)
            mhc.post(X, Y, Hs[l], out=Xn)
            X, Xn = Xn, X
        return X

    def fused_layers(cp=params, kc=kw):
        X, Xn = XA, XB
        mhc.pre(X, cp[0][0], cp[0][1], h=h, H=Hs[0], workspace=ws, **kc)
        for l in range(L - 1):
            mhc.gelu_half(h, out=Y)
            mhc.post_pre(X, Y, Hs[l], cp[l + 1][0], cp[l + 1][1], out=Xn, h=h, H_next=Hs[l + 1],
                         workspace=ws, **kc)
            X, Xn = Xn, X
        mhc.gelu_half(h, out=Y)
        mhc.post(X, Y, Hs[L - 1], out=Xn)
        return Xn

    def fused():
        XA.copy_(X0)
        return fused_layers()

    out = {"workload": w.name, "layers": L}
    for name, fn in (("separate", separate), ("fused_post_pre", fused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        out[name] = {"total_ms": ms, "per_layer_us": ms * 1e3 / L}
    # The fused chain captured into one HIP graph (the state copy stays
    # outside): every replay must give the eager chain's final state and maps.
    Xf = fused()
    torch.cuda.synchronize()
    X_ref, Hs_ref = Xf.clone(), Hs.clone()
    graph = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    XA.copy_(X0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gs):
        fused_layers()
    for rnd in range(reps):
        XA.copy_(X0)
        Hs.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(Xf, X_ref) and torch.equal(Hs, Hs_ref)):
            raise SystemExit(f"stack graph replay {rnd} differs from the eager chain")
    # Timed like the eager chain: back to back, the state copy in front of each.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        XA.copy_(X0)
        graph.replay()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    out["fused_post_pre_hip_graph"] = {"total_ms": ms, "per_layer_us": ms * 1e3 / L,
                                       "note": "state copy outside the graph, each replay checked against the eager "
                                               "chain, then replays timed back to back"}

    mhc.amax(Hs, n, out_amax=amax, want_all=False)
    a = amax.cpu().numpy()
    out["amax"] = {"max": float(a.max()), "mean": float(a.mean()), "min": float(a.min())}

    # Contrast: the HC form of the maps on the HC stack workload (b_res =
    # I + N(0, 0.3) per layer, as in the pages' NumPy demo), and the mHC maps
    # on the same biases; per-token composite Amax of each.
    wc = synth.WORKLOADS["hc_stack60_bf16_T4096_d2560"]
    cparams = [tuple(dev(a) for a in synth.make_params(wc, layer=l)) for l in range(L)]
    X0c = dev(synth.make_state(wc))
    contrast = {"workload": wc.name}
    for name, maps in (("hc", mhc.MAPS_HC), ("mhc_same_biases", mhc.MAPS_MHC)):
        kc = dict(alpha=wc.alpha, eps=wc.eps, t_max=wc.t_max, maps=maps)
        XA.copy_(X0c)
        fused_layers(cparams, kc)
        mhc.amax(Hs, n, out_amax=amax, want_all=False)
        a = amax.cpu().numpy()
        contrast[name] = {"amax_max": float(a.max()), "amax_median": float(np.median(a)), "amax_min": float(a.min())}
    out["contrast"] = contrast
    return out


def time_post_pre(mhc, torch, w, X, Y, H, phi, bias, reps, stream):
    """Layer l's mhc_post fused with layer l+1's mhc_pre at the workload's
    shape, both forms, per call (HIP events at the ends of `reps` calls, the
    median of three rounds).
    GB/s on the least bytes such a fused layer moves: X_l and Y read, X_{l+1}
    and h written, the maps read and written (80 KiB per token at n = 4,
    d = 4096, bf16)."""
    T, n, d = X.shape
    m = n * n + 2 * n
    sb = X.element_size()
    least = T * (2 * n * d * sb + 2 * d * sb + 2 * m * 4)
    Xo, h2, H2 = torch.empty_like(X), torch.empty_like(Y), torch.empty_like(H)
    ws = torch.zeros(mhc.pre_workspace_size(T, n, d, mhc.MHC_BF16 if sb == 2 else mhc.MHC_FP32), dtype=torch.uint8,
                     device=X.device)
    out = {"least_bytes_per_token": least // T, "forms": {}}
    forms = [("one-pass", mhc.PRE_ONE_PASS), ("two-pass", mhc.PRE_TWO_PASS)]
    calls = {}
    for name, algo in forms:
        def call(algo=algo):
            return mhc.post_pre_ex(X, Y, H, phi, bias, algo, alpha=w.alpha, eps=w.eps, t_max=w.t_max, out=Xo, h=h2,
                                   H_next=H2, workspace=ws, stream=stream)[3]
        try:
            for _ in range(3):
                call()
            calls[name] = call
        except mhc.MhcError:
            out["forms"][name] = None
    # Three rounds, the order of the forms alternating, and each form's median
    # round: the first calls after start-up run slower, whichever form they are.
    runs = {name: [] for name in calls}
    for rnd in range(3):
        for name in (list(calls) if rnd % 2 == 0 else list(calls)[::-1]):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record(stream)
            for _ in range(reps):
                calls[name]()
            ev[1].record(stream)
            torch.cuda.synchronize()
            runs[name].append(ev[0].elapsed_time(ev[1]) / reps * 1e3)
    for name, v in runs.items():
        us = sorted(v)[len(v) // 2]
        out["forms"][name] = {"avg_us": us, "rounds_us": v, "GBps_on_least_bytes": least / (us * 1e-6) / 1e9,
                              "frac_of_peak": least / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
    out["auto_form"] = {1: "two-pass", 2: "one-pass"}.get(
        mhc.post_pre_ex(X, Y, H, phi, bias, mhc.PRE_AUTO, alpha=w.alpha, eps=w.eps, t_max=w.t_max, out=Xo, h=h2,
                        H_next=H2, workspace=ws, stream=stream)[3])
    torch.cuda.synchronize()
    return out


def traffic_bytes(path, workload, entry):
    """HBM bytes per launch of an entry point measured with rocprofv3
    counters, or None when absent or when the kernel source changed since."""
    import hashlib
    try:
        with open(path) as f:
            rec = json.load(f).get(workload, {}).get(entry)
        if not rec or not rec.get("valid", False):
            return None
        h = hashlib.sha256()
        for p in rec["sources"]:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
        return rec["bytes_per_launch"] if h.hexdigest()[:16] == rec["source_sha256_16"] else None
    except (OSError, ValueError, KeyError):
        return None


def time_small_t(mhc, torch, reps=100):
    """Per-call latency of mhc_pre at decode-sized T (the small-T split-K
    form), on random inputs of the layer shapes: n = 4 bf16 at d = 4096 and
    d = 2048, and the fp32 T = 64, d = 256 workload."""
    out = []
    for d, dt, T in ((4096, torch.bfloat16, 1), (4096, torch.bfloat16, 16), (4096, torch.bfloat16, 64),
                     (2048, torch.bfloat16, 64), (256, torch.float32, 64)):
        n, m = 4, 24
        g = torch.Generator(device="cuda").manual_seed(T * 7 + d)
        X = torch.randn(T, n, d, device="cuda", generator=g).to(dt)
        phi = torch.randn(n * d, m, device="cuda", generator=g) * 0.02
        bias = torch.randn(m, device="cuda", generator=g) * 0.1
        code = 1 if dt == torch.bfloat16 else 0
        ws = torch.empty(mhc.pre_workspace_size(T, n, d, code), dtype=torch.uint8, device="cuda")
        h = torch.empty((T, d), dtype=dt, device="cuda")
        H = torch.empty((T, m), device="cuda")
        for _ in range(10):
            mhc.pre_ex(X, phi, bias, 0, h=h, H=H, workspace=ws)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            mhc.pre_ex(X, phi, bias, 0, h=h, H=H, workspace=ws)
        ev[1].record()
        torch.cuda.synchronize()
        eager_us = ev[0].elapsed_time(ev[1]) / reps * 1e3
        # The same calls captured into a HIP graph (how a decode loop would
        # run them): 20 calls per graph, replayed; every replay's h and H
        # must equal the eager call's bits.
        h_ref, H_ref = h.clone(), H.clone()
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        per_graph = 20
        with torch.cuda.graph(graph, stream=s):
            for _ in range(per_graph):
                mhc.pre_ex(X, phi, bias, 0, h=h, H=H, workspace=ws)
        graph_us = None
        for rnd in range(3):
            h.zero_()
            H.zero_()
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(reps // per_graph):
                graph.replay()
            ev[1].record()
            torch.cuda.synchronize()
            if not (torch.equal(h, h_ref) and torch.equal(H, H_ref)):
                raise SystemExit(f"graph replay {rnd} differs from the eager call at T={T} d={d}")
            us = ev[0].elapsed_time(ev[1]) / ((reps // per_graph) * per_graph) * 1e3
            graph_us = us if graph_us is None else min(graph_us, us)
        out.append({"shape": f"T={T} n=4 d={d} {'bf16' if code else 'fp32'}", "us": eager_us,
                    "us_in_hip_graph": graph_us})
    return out


def time_small_configs(mhc, torch, reps=50):
    """The forward step (mhc_pre -> Y given -> mhc_post -> mhc_amax) on the
    two smaller single-layer workloads, T = 64, d = 256 fp32 and T = 4096,
    d = 2048 bf16, with the generator's inputs: per step and tokens/s."""
    import numpy as np

    import synth
    out = []
    for name in ("layer_fp32_T64_d256", "layer_bf16_T4096_d2048"):
        w = synth.WORKLOADS[name]

        def dev(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
            return torch.from_numpy(a).cuda()

        X, Y = dev(synth.make_state(w)), dev(synth.make_sublayer_out(w))
        phi, bias = (dev(a) for a in synth.make_params(w))
        T, n, d, m = w.T, w.n, w.d, w.m
        h = torch.empty((T, d), dtype=X.dtype, device="cuda")
        H = torch.empty((T, m), dtype=torch.float32, device="cuda")
        Xo = torch.empty_like(X)
        amax = torch.empty(T, dtype=torch.float32, device="cuda")
        ws = torch.empty(max(16, mhc.pre_workspace_size(T, n, d, w.dtype)), dtype=torch.uint8, device="cuda")

        def step():
            mhc.pre(X, phi, bias, alpha=w.alpha, eps=w.eps, t_max=w.t_max, h=h, H=H, workspace=ws)
            mhc.post(X, Y, H, out=Xo)
            mhc.amax(H.view(1, T, m), n, out_amax=amax, want_all=False)

        for _ in range(10):
            step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            step()
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) / reps * 1e3
        # The same steps captured into a HIP graph (10 steps per graph),
        # replayed: the device time without the host's per-call overhead,
        # which bounds the eager steps of the small workload.  Every
        # replay's outputs must equal the eager step's bits.
        refs = [t.clone() for t in (h, H, Xo, amax)]
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        per_graph = 10
        with torch.cuda.graph(graph, stream=s):
            for _ in range(per_graph):
                step()
        graph_us = None
        for rnd in range(3):
            for t in (h, H, Xo, amax):
                t.zero_()
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(reps // per_graph):
                graph.replay()
            ev[1].record()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip((h, H, Xo, amax), refs)):
                raise SystemExit(f"graph replay {rnd} of the {name} step differs from the eager step")
            g_us = ev[0].elapsed_time(ev[1]) / ((reps // per_graph) * per_graph) * 1e3
            graph_us = g_us if graph_us is None else min(graph_us, g_us)
        out.append({"workload": name, "us_per_step": us, "tokens_per_s": T / (us * 1e-6),
                    "us_per_step_in_hip_graph": graph_us, "tokens_per_s_in_hip_graph": T / (graph_us * 1e-6)})
    return out


def time_n8(mhc, torch, T=16384, d=4096, reps=10):
    """mhc_pre and mhc_post at n = 8 streams (m = 80, bf16, random inputs of
    the layer's distributions), per call, with their algorithmic GB/s."""
    n, m = 8, 80
    g = torch.Generator(device="cuda").manual_seed(88)
    X = torch.randn(T, n, d, device="cuda", generator=g).to(torch.bfloat16)
    Y = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
    phi = torch.randn(n * d, m, device="cuda", generator=g) * 0.02
    bias = torch.randn(m, device="cuda", generator=g) * 0.1
    ws = torch.empty(mhc.pre_workspace_size(T, n, d, 1), dtype=torch.uint8, device="cuda")
    h = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    H = torch.empty((T, m), device="cuda")
    Xo = torch.empty_like(X)
    out = {"shape": f"T={T} n=8 d={d} bf16"}
    calls = (("mhc_pre", lambda: mhc.pre(X, phi, bias, h=h, H=H, workspace=ws), T * n * d * 2 + T * d * 2 + T * m * 4),
             ("mhc_post", lambda: mhc.post(X, Y, H, out=Xo), 2 * T * n * d * 2 + T * d * 2 + T * (n * n + n) * 4))
    for name, fn, nbytes in calls:
        for _ in range(3):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) / reps * 1e3
        out[name] = {"avg_us": us, "GBps": nbytes / us / 1e3}
    return out


def load_bench_lib():
    """libmhc_bench.so: the streaming-copy reference kernel (built with libmhc)."""
    import ctypes
    path = os.path.join(ROOT, "mhc_hyper_connections_amd", "libmhc_bench.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.mhc_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mhc_bench_copy.restype = ctypes.c_int
    return lib


def time_copy(torch, src, dst, stream, reps=10):
    """GB/s (read + write) of the streaming copy of src into dst, HIP events on `stream`."""
    import ctypes
    lib = load_bench_lib()
    nbytes = src.numel() * src.element_size()
    s = ctypes.c_void_p(stream.cuda_stream)

    def run():
        if lib.mhc_bench_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, s) != 0:
            raise SystemExit("mhc_bench_copy failed")

    for _ in range(3):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        run()
    ev[1].record(stream)
    torch.cuda.synchronize()
    if not torch.equal(src, dst):
        raise SystemExit("the streaming copy did not reproduce its source")
    return 2 * nbytes * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9


def cpu_baseline(w, seconds_target=15.0):
    """The oracle (single-threaded C++, double) on the first tokens of the
    same workload: mhc_pre + mhc_post per token."""
    import numpy as np

    import oracle
    import synth
    o = oracle.load()
    phi, bias = synth.make_params(w)
    probe = 8
    Xs, Ys = synth.make_state(w, probe), synth.make_sublayer_out(w, probe)
    t0 = time.perf_counter()
    r = o.pre(Xs, phi, bias, w.alpha, eps=w.eps, t_max=w.t_max)
    o.post(Xs, Ys, r["H"].astype(np.float32))
    per_tok = (time.perf_counter() - t0) / probe
    ntok = int(max(probe, min(w.T, seconds_target / max(per_tok, 1e-9))))
    Xs, Ys = synth.make_state(w, ntok), synth.make_sublayer_out(w, ntok)
    t0 = time.perf_counter()
    r = o.pre(Xs, phi, bias, w.alpha, eps=w.eps, t_max=w.t_max)
    o.post(Xs, Ys, r["H"].astype(np.float32))
    dt = time.perf_counter() - t0
    host_cores = os.cpu_count() or 1
    try:
        host_cores_usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        host_cores_usable = host_cores
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    out = {"value": ntok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"first {ntok} of {w.T} tokens of {w.name}, mhc_pre + mhc_post, fp64, "
                     f"{dt:.1f} s on one host thread",
           "host_cores": host_cores, "host_cores_usable": host_cores_usable, "cpu_model": cpu_model}
    # The same oracle calls sharded over tokens on host threads (the calls
    # release the GIL).  16 threads at most: the share of the host's cores
    # that goes with one GPU on a multi-GPU node (the host may show more).
    import concurrent.futures as cf
    threads = max(1, min(16, host_cores_usable))
    bounds = [(k * ntok // threads, (k + 1) * ntok // threads) for k in range(threads)]

    def run(b):
        a, e = b
        if e <= a:
            return
        rr = o.pre(Xs[a:e], phi, bias, w.alpha, eps=w.eps, t_max=w.t_max)
        o.post(Xs[a:e], Ys[a:e], rr["H"].astype(np.float32))

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, bounds))
    dtm = time.perf_counter() - t0
    out["all_cores"] = {"value": ntok / dtm, "unit": "tokens/s", "cores": threads,
                        "sample": f"the same {ntok} tokens split over {threads} host threads, {dtm:.2f} s",
                        "why_16": "at most 16 threads: one GPU's share of the host's cores"}
    return out


# ---- rocprofv3 results -> profiles/ ------------------------------------------
# Which kernels make up each entry point (substrings of the demangled names).
ENTRY_KERNELS = {
    "mhc_pre": ["pre_one_pass_kernel<4, false, false>", "pre_one_pass_fallback_kernel<4, false, false>"],   # AUTO's form
    "mhc_pre_two_pass": ["pre_partial_kernel<mhc::BF16, 4, 2, 0, 8, false>", "pre_finish_kernel<mhc::BF16, 4, false, 4>"],
    "mhc_post": ["post_tile_kernel<mhc::BF16, 4>"],
    "mhc_post_pre_one_pass": ["pre_one_pass_kernel<4, false, true>", "pre_one_pass_fallback_kernel<4, false, true>"],
    "mhc_post_pre_two_pass": ["pre_partial_kernel<mhc::BF16, 4, 1, 2, 8, false>",
                              "pre_finish_kernel<mhc::BF16, 4, false, 4>"],
    "mhc_amax": ["amax_kernel<4>"],
    "mhc_post_bwd": ["post_bwd_tile_kernel<mhc::BF16, 4, true>", "post_bwd_reduce_kernel<4>"],
    "mhc_pre_bwd": ["pre_partial_kernel<mhc::BF16, 4, 1, 1, 8, false>", "pre_bwd_token_kernel<4, true>",
                    "pre_bwd_apply_mfma_kernel<4, false>", "reduce_grads_kernel"],
    # the whole-dX pair: mhc_post_bwd with dX NULL, then mhc_pre_bwd_ex with G
    "mhc_post_bwd_without_dX": ["post_bwd_tile_kernel<mhc::BF16, 4, false>", "post_bwd_reduce_kernel<4>"],
    "mhc_pre_bwd_ex_with_G": ["pre_partial_kernel<mhc::BF16, 4, 1, 1, 8, false>", "pre_bwd_token_kernel<4, true>",
                              "pre_bwd_apply_mfma_kernel<4, true>", "reduce_grads_kernel"],
}
ENTRY_SOURCES = {
    "mhc_pre": ["pre_fused.hip", "pre_common.hpp", "device.hpp"],
    "mhc_pre_two_pass": ["pre.hip", "pre_common.hpp", "device.hpp"],
    "mhc_post": ["post.hip", "device.hpp"],
    "mhc_post_pre_one_pass": ["pre_fused.hip", "pre_common.hpp", "device.hpp"],
    "mhc_post_pre_two_pass": ["pre.hip", "pre_common.hpp", "device.hpp"],
    "mhc_amax": ["amax.hip", "device.hpp"],
    "mhc_post_bwd": ["bwd.hip", "device.hpp"],
    "mhc_pre_bwd": ["bwd.hip", "pre.hip", "pre_common.hpp", "device.hpp"],
    "mhc_post_bwd_without_dX": ["bwd.hip", "device.hpp"],
    "mhc_pre_bwd_ex_with_G": ["bwd.hip", "pre.hip", "pre_common.hpp", "device.hpp"],
}
COPY_KERNEL = "stream_copy_kernel"  # libmhc_bench's streaming copy of the 512 MiB state: one read, one write


def _db_rows(path, query):
    import sqlite3
    with sqlite3.connect(path) as con:
        return list(con.execute(query))


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def _working_median(vals):
    """Median over the dispatches of the workload's size: those within half of
    the largest.  The counter runs also launch the same kernels on smaller
    shapes (the smaller single-layer workloads, decode-sized calls), and the
    headline workload is the largest; a kernel that always returns at once,
    like the single pass's fallback kernel, keeps all of its dispatches."""
    top = max(vals)
    return _median([v for v in vals if v >= 0.5 * top])


def _counter_per_kernel(path, counter):
    per = {}
    for name, cname, val in _db_rows(path, "select kernel_name, counter_name, value from counters_collection"):
        if cname == counter:
            per.setdefault(name, []).append(float(val))
    return per


def write_traffic(fetch_db, write_db, out_path, workload="layer_bf16_T16384_d4096"):
    """HBM bytes per launch of each entry point from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the plain copy of the state (known: 512 MiB read and
    512 MiB written).  Records the sources' hash so a changed kernel voids it."""
    import hashlib
    fetch = _counter_per_kernel(fetch_db, "FETCH_SIZE")
    write = _counter_per_kernel(write_db, "WRITE_SIZE")
    copy_bytes = 512 * 1024 * 1024

    def copy_median(per):
        # The 512 MiB copy's dispatches: torch's small multiplies (input
        # set-up) run the same kernel, so keep the dispatches near the largest.
        vals = [v for k, vs in per.items() if COPY_KERNEL in k for v in vs]
        if not vals:
            raise SystemExit("the plain-copy kernel is missing from the counter runs")
        top = max(vals)
        return _median([v for v in vals if v >= 0.5 * top])
    fetch_scale = copy_bytes / (copy_median(fetch) * 1024)
    write_scale = copy_bytes / (copy_median(write) * 1024)
    entries = {}
    for entry, pats in ENTRY_KERNELS.items():
        rb = wb = 0.0
        found = 0
        for pat in pats:
            kf = [k for k in fetch if pat in k]
            kw = [k for k in write if pat in k]
            if kf and kw:
                found += 1
                rb += _working_median(fetch[kf[0]]) * 1024 * fetch_scale
                wb += _working_median(write[kw[0]]) * 1024 * write_scale
        if found != len(pats):
            continue
        h = hashlib.sha256()
        srcs = [os.path.join("mhc_hyper_connections_amd", "csrc", f) for f in ENTRY_SOURCES[entry]]
        for p in srcs:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
        entries[entry] = {"bytes_per_launch": int(rb + wb), "read_bytes": int(rb), "write_bytes": int(wb),
                          "kernels": pats, "source_sha256_16": h.hexdigest()[:16], "sources": srcs, "valid": True}
    doc = {"_note": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, median over "
                    "the dispatches that did the work), "
                    "each scaled by what the same counter reads for a plain copy of the 512 MiB state "
                    f"(FETCH_SIZE x {fetch_scale:.5f}, WRITE_SIZE x {write_scale:.5f}). Valid while the "
                    "sources' hash matches.",
           "fetch_scale": fetch_scale, "write_scale": write_scale, workload: entries}
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
    return doc


def summarize_trace(stats_db):
    """Markdown table of a rocprofv3 --kernel-trace --stats run (per-kernel average durations, over all
    dispatches and over those within half of the kernel's longest, i.e. its largest shape).  A kernel
    whose dispatches fall into a group under 8 us and a group over 40 us is listed twice (the short
    ones returned at once)."""
    rows = _db_rows(stats_db, "select name, duration from kernels")       # duration in ns
    total = sum(d for _, d in rows) or 1
    groups = {}
    for name, dur in rows:
        groups.setdefault(name, []).append(dur / 1000.0)
    entries = []
    for name, durs in groups.items():
        short = name.replace("void ", "").replace("mhc::(anonymous namespace)::", "").split("(")[0]
        if COPY_KERNEL in name:
            parts = [("stream_copy_kernel (plain copy of the state, 1 read + 1 write of 512 MiB)", durs)]
        elif "mhc::" in name and min(durs) < 8.0 and max(durs) > 40.0:
            parts = [(short, [d for d in durs if d >= 8.0]),
                     (short + " — dispatches that returned at once", [d for d in durs if d < 8.0])]
        else:
            parts = [(short, durs)]
        for label, ds in parts:
            if ds:
                # the dispatches of the largest shape (a kernel also runs on smaller ones: the bench's smaller
                # workloads, the alone and in-step timings share the headline shape)
                big = [x for x in ds if x >= 0.5 * max(ds)]
                entries.append((label, len(ds), sum(ds) / len(ds), 100.0 * sum(ds) * 1000.0 / total, big))
    entries.sort(key=lambda e: -e[3])
    lines = ["| kernel | calls | average us | share of GPU time | calls within half of the longest | their average us |",
             "|---|---|---|---|---|---|"]
    for label, calls, avg, pct, big in ((e[0], e[1], e[2], e[3], e[4]) for e in entries):
        lines.append(f"| `{label[:110]}` | {calls} | {avg:.1f} | {pct:.1f}% | {len(big)} | {sum(big) / len(big):.1f} |")
    return "\n".join(lines)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--write-traffic":
        doc = write_traffic(sys.argv[2], sys.argv[3], sys.argv[4] if len(sys.argv) > 4 else
                            os.path.join(ROOT, "profiles", "hbm_traffic.json"))
        print(json.dumps(doc, indent=1))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        print(summarize_trace(sys.argv[2]))
        return
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-s", type=float, default=0.2,
                    help="seconds of untimed steps before the warm-up steps (0: none, as in the profiler runs)")
    ap.add_argument("--workload", default="layer_bf16_T16384_d4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-stack", action="store_true", help="skip the 60-layer stack timing")
    ap.add_argument("--stack-only", action="store_true",
                    help="time only the 60-layer stack (for a kernel trace of it); prints its JSON and exits")
    ap.add_argument("--post-pre-only", action="store_true",
                    help="time only mhc_post_pre's two forms at the workload's shape, after the plain copy (for "
                         "counter runs); prints their JSON and exits")
    ap.add_argument("--pre-algo", type=int, default=0, choices=[0, 1, 2],
                    help="mhc_pre form: 0 auto, 1 two-pass, 2 one-pass")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters (optional)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the forward needs no "
              f"communication: tokens shard across GPUs with phi replicated).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mhc_hyper_connections_amd as mhc
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.stack_only:
        mhc.load_library()
        print(json.dumps(time_stack(mhc, torch, reps=3, warmup=1)))
        return 0
    mhc.load_library()
    # Decode-sized calls first, on a fresh allocator: timed after the large
    # workload's buffers were allocated, one of these shapes (T = 64,
    # d = 4096) measured 23 us per call against 13 us alone, for a reason not
    # yet found; the number reported is the isolated per-call latency.
    # No cyclic garbage collection while timing: a full collection with torch
    # loaded took up to 34 ms of host time here, long enough to drain the
    # GPU's queue and add a gap to one step's interval (one backward step
    # measured 61 ms against a 590 us median).
    gc.collect()
    gc.disable()
    small_t = time_small_t(mhc, torch)
    torch.cuda.empty_cache()
    w = synth.WORKLOADS[args.workload]
    if w.layers != 1:
        raise SystemExit("bench.py times single-layer workloads")
    T, n, d = w.T, w.n, w.d
    sbytes = 2 if w.dtype == synth.BF16 else 4
    log(f"workload {w.name}: T={T} n={n} d={d} {'bf16' if sbytes == 2 else 'fp32'}; generating inputs")

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    X = dev(synth.make_state(w))
    Y = dev(synth.make_sublayer_out(w))
    phi, bias = (dev(a) for a in synth.make_params(w))
    m = n * n + 2 * n
    h = torch.empty((T, d), dtype=X.dtype, device="cuda")
    H = torch.empty((T, m), dtype=torch.float32, device="cuda")
    Xo = torch.empty_like(X)
    amax = torch.empty(T, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, mhc.pre_workspace_size(T, n, d, w.dtype)), dtype=torch.uint8, device="cuda")
    H1 = H.view(1, T, m)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log("inputs resident; warming up")

    algo_used = [None]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        _, _, algo_used[0] = mhc.pre_ex(X, phi, bias, args.pre_algo, alpha=w.alpha, eps=w.eps, t_max=w.t_max,
                                        h=h, H=H, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        mhc.post(X, Y, H, out=Xo, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        mhc.amax(H1, n, out_amax=amax, want_all=False, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    # A plain copy of known size (X -> X', one read and one write of the
    # state) by a hand-written streaming kernel: the practical HBM ceiling,
    # and the reference that scales the rocprofv3 byte counters.
    copy_GBps = time_copy(torch, X, Xo, stream)
    log(f"plain copy of the state (stream_copy_kernel): {copy_GBps:.0f} GB/s")
    if args.post_pre_only:
        step()
        pp = time_post_pre(mhc, torch, w, X, Y, H, phi, bias, args.steps, stream)
        print(json.dumps({"copy_GBps": copy_GBps, "post_pre": pp}), flush=True)
        return 0

    # The first few milliseconds of steps after start-up run several percent
    # slower on MI355X, whatever the kernels: before the W warm-up steps the
    # step runs, untimed, for at least --settle-s seconds (0.2 by default).
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n_settle += 20
    log(f"settled: {n_settle} untimed steps in {time.perf_counter() - t_settle:.2f} s")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    # The timed region: K steps back to back with HIP events (on the stream
    # every call is launched on) only at its two ends, bracketed by device
    # synchronisations.  `value` and `ms_per_step` come from it.
    log(f"timing {K} steps")
    bev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    bev[0].record(stream)
    for k in range(K):
        step()
    bev[1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = bev[0].elapsed_time(bev[1]) / K
    tokens_per_s = T / (ms_step * 1e-3)
    # The per-entry-point breakdown: the same K steps again, right after,
    # with an event between every two calls.  Each event splits the stream
    # (about 25 us per step on MI355X), so these steps are longer than the
    # timed ones; the durations of the calls themselves are what is used.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        step(evs[k])
    torch.cuda.synchronize()
    ms_step_events = evs[0][0].elapsed_time(evs[K - 1][3]) / K
    per = {"mhc_pre": [], "mhc_post": [], "mhc_amax": []}
    for e in evs:
        per["mhc_pre"].append(e[0].elapsed_time(e[1]))
        per["mhc_post"].append(e[1].elapsed_time(e[2]))
        per["mhc_amax"].append(e[2].elapsed_time(e[3]))
    # Each entry point alone: K calls back to back on the same inputs, HIP
    # events only at the ends.  This is the average duration of one call
    # (its kernels and the gaps between them) with nothing between calls.
    alone_calls = {
        "mhc_pre": lambda: mhc.pre_ex(X, phi, bias, args.pre_algo, alpha=w.alpha, eps=w.eps, t_max=w.t_max, h=h,
                                      H=H, workspace=ws, stream=stream),
        "mhc_post": lambda: mhc.post(X, Y, H, out=Xo, stream=stream),
        "mhc_amax": lambda: mhc.amax(H1, n, out_amax=amax, want_all=False, stream=stream),
    }
    alone = {}
    for name, call in alone_calls.items():
        for _ in range(3):
            call()
        aev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        aev[0].record(stream)
        for _ in range(K):
            call()
        aev[1].record(stream)
        torch.cuda.synchronize()
        alone[name] = aev[0].elapsed_time(aev[1]) / K
    algo = algorithmic_bytes(T, n, d, sbytes)
    step_bytes = sum(algo.values())
    kernels = {}
    for name, ts in per.items():
        avg_ms = alone[name]
        kernels[name] = {"avg_us": avg_ms * 1e3,
                         "in_step_with_events_avg_us": float(np.mean(ts)) * 1e3,
                         "in_step_with_events_median_us": float(np.median(ts)) * 1e3,
                         "algorithmic_bytes": algo[name],
                         "GBps": algo[name] / (avg_ms * 1e-3) / 1e9,
                         "frac_of_peak": algo[name] / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "share_of_step": avg_ms / ms_step}
    # The roofline is reported for the bottleneck: of the entry points that
    # take at least a quarter of the step, the one furthest below the HBM
    # peak (mhc_pre here; mhc_post takes about as long but runs nearer peak).
    major = [k for k in kernels if kernels[k]["share_of_step"] >= 0.25] or list(kernels)
    dominant = min(major, key=lambda k: kernels[k]["frac_of_peak"])
    form_key = {"mhc_pre": "mhc_pre" if algo_used[0] == 2 else "mhc_pre_two_pass"}
    traffic = traffic_bytes(args.traffic_json, w.name, form_key.get(dominant, dominant))
    kd = kernels[dominant]
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": kd["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": kd["GBps"] / HBM_PEAK_GBPS, "traffic": traffic,
                "algorithmic_bytes_per_launch": kd["algorithmic_bytes"], "avg_launch_us": kd["avg_us"],
                "choice": "the entry point furthest below peak among those taking >= 25% of the step"}
    log(f"{ms_step * 1e3:.1f} us/step ({ms_step_events * 1e3:.1f} us with an event between calls), "
        f"{tokens_per_s / 1e6:.2f} M tokens/s; "
        + ", ".join(f"{k} {v['avg_us']:.1f} us ({v['GBps']:.0f} GB/s)" for k, v in kernels.items()))

    # The other form of mhc_pre on the same inputs, for reference.
    # The two forms in three rounds, their order alternating, each form's
    # median round (the first calls after an idle moment run slower).
    forms = {}
    pre_calls = {}
    for form_algo, name in ((2, "one-pass"), (1, "two-pass")):
        def pcall(form_algo=form_algo):
            mhc.pre_ex(X, phi, bias, form_algo, alpha=w.alpha, eps=w.eps, t_max=w.t_max, h=h, H=H, workspace=ws,
                       stream=stream)
        try:
            for _ in range(3):
                pcall()
            pre_calls[name] = pcall
        except mhc.MhcError:
            forms[name] = None
    pre_runs = {name: [] for name in pre_calls}
    for rnd in range(3):
        for name in (list(pre_calls) if rnd % 2 == 0 else list(pre_calls)[::-1]):
            fev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            fev[0].record(stream)
            for _ in range(max(5, K // 2)):
                pre_calls[name]()
            fev[1].record(stream)
            torch.cuda.synchronize()
            pre_runs[name].append(fev[0].elapsed_time(fev[1]) / max(5, K // 2) * 1e3)
    for name, v in pre_runs.items():
        us = sorted(v)[len(v) // 2]
        forms[name] = {"avg_us": us, "rounds_us": v,
                       "GBps": algorithmic_bytes(T, n, d, sbytes)["mhc_pre"] / (us * 1e-6) / 1e9}
    log("mhc_pre forms: " + ", ".join(f"{k} {v['avg_us']:.1f} us" for k, v in forms.items() if v))

    post_pre = time_post_pre(mhc, torch, w, X, Y, H, phi, bias, max(5, K // 2), stream)
    log("mhc_post_pre (layer l's post + layer l+1's pre) at this shape: " + ", ".join(
        f"{k} {v['avg_us']:.1f} us ({v['GBps_on_least_bytes']:.0f} GB/s on {post_pre['least_bytes_per_token']} B/token)"
        for k, v in post_pre["forms"].items() if v) + f"; AUTO takes {post_pre['auto_form']}")
    n8 = time_n8(mhc, torch)
    small_cfg = time_small_configs(mhc, torch)
    log("smaller layers (forward step; in a HIP graph): " + ", ".join(
        f"{r['workload']} {r['us_per_step']:.1f} us ({r['tokens_per_s'] / 1e6:.2f} M tokens/s; "
        f"{r['us_per_step_in_hip_graph']:.1f} us)" for r in small_cfg))
    log(f"n = 8 ({n8['shape']}): mhc_pre {n8['mhc_pre']['avg_us']:.1f} us ({n8['mhc_pre']['GBps']:.0f} GB/s), "
        f"mhc_post {n8['mhc_post']['avg_us']:.1f} us ({n8['mhc_post']['GBps']:.0f} GB/s)")
    log("mhc_pre at small T (split-K form, per call; in a HIP graph): " +
        ", ".join(f"{r['shape']} {r['us']:.1f} us ({r['us_in_hip_graph']:.1f} us)" for r in small_t))

    backward = None
    if not args.no_backward:
        log("timing the backward (mhc_post_bwd + mhc_pre_bwd)")
        backward = time_backward(mhc, torch, w, X, Y, phi, bias, H, max(5, K // 2), 3, stream)
        if backward is not None:
            bwd_us = min(backward["total_us"], backward["whole_dX"]["total_us"])
            backward["fwd_bwd_tokens_per_s"] = T / ((ms_step * 1e3 + bwd_us) * 1e-6)
            log(f"backward: post_bwd {backward['mhc_post_bwd']['avg_us']:.1f} us, pre_bwd "
                f"{backward['mhc_pre_bwd']['avg_us']:.1f} us, together {backward['total_us']:.1f} us: "
                f"{backward['GBps']:.0f} GB/s on the least bytes ({100 * backward['frac_of_peak']:.0f}% of peak); "
                f"whole-dX pair {backward['whole_dX']['total_us']:.1f} us (post_bwd without dX "
                f"{backward['whole_dX']['mhc_post_bwd_without_dX_us']:.1f} us, pre_bwd_ex "
                f"{backward['whole_dX']['mhc_pre_bwd_ex_us']:.1f} us, {100 * backward['whole_dX']['frac_of_peak']:.0f}% of peak)"
                + f"; post_bwd without workspace {backward['mhc_post_bwd_scratch_free_us']:.1f} us")

    stack = None
    if not args.no_stack:
        log("timing the 60-layer stack (separate entry points, then mhc_post_pre)")
        stack = time_stack(mhc, torch)
        log(f"stack: separate {stack['separate']['total_ms']:.2f} ms "
            f"({stack['separate']['per_layer_us']:.1f} us/layer), fused {stack['fused_post_pre']['total_ms']:.2f} ms "
            f"({stack['fused_post_pre']['per_layer_us']:.1f} us/layer), fused in a HIP graph "
            f"{stack['fused_post_pre_hip_graph']['total_ms']:.2f} ms "
            f"({stack['fused_post_pre_hip_graph']['per_layer_us']:.1f} us/layer); amax max {stack['amax']['max']:.6f}; "
            f"contrast: HC amax median {stack['contrast']['hc']['amax_median']:.1f}, mHC on the same biases "
            f"{stack['contrast']['mhc_same_biases']['amax_median']:.4f}")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w)
        log(f"oracle: {cpu['value']:.1f} tokens/s ({cpu['sample']}); on {cpu['all_cores']['cores']} threads "
            f"{cpu['all_cores']['value']:.1f} tokens/s")

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sbytes == 2 else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "n": n, "d": d, "t_max": w.t_max,
                   "step": "mhc_pre + mhc_post + mhc_amax (one layer), Y given",
                   "mhc_pre_form": {1: "two-pass", 2: "one-pass"}.get(algo_used[0], str(algo_used[0])),
                   "parallelism": "single GPU"},
        "achieved_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "achieved_frac_of_hbm_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "copy_GBps": copy_GBps,
        "copy_kernel": "stream_copy_kernel (libmhc_bench.so): 16-byte non-temporal loads and stores, "
                       "4 KiB per workgroup, of the 512 MiB state into a second buffer",
        "timing": "value and ms_per_step: K steps with HIP events only at the two ends; kernels[*].avg_us: K "
                  "calls of that entry point alone, events only at the ends; in_step_with_events_*: the K steps "
                  "again with an event between calls (ms_per_step_with_events)",
        "ms_per_step_with_events": ms_step_events,
        "step_roofline": {"bound": "hbm", "achieved": step_bytes / (ms_step * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "target_frac": 0.70},
        "wall_s_timed_region": t_wall,
        "roofline": roofline,
        "kernels": kernels,
        "mhc_pre_forms": forms,
        "small_t": small_t,
        "post_pre": post_pre,
        "n8": n8,
        "smaller_layers": small_cfg,
        "backward": backward,
        "stack": stack,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
