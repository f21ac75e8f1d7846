"""mhc_hyper_connections_amd: the mHC layer forward on AMD Instinct MI355X (gfx950).

The product is ``libmhc.so``, a C-ABI library of hand-written HIP kernels
(declared in ``include/mhc.h``).  This package is its thin Python binding:

    h, H = mhc.pre(X, phi, bias, alpha=(a_pre, a_res, a_post), eps=1e-6, t_max=20)
    Y    = F(h)                                   # the caller's sublayer
    Xn   = mhc.post(X, Y, H)                      # or out=X for in place
    Xn, h2, H2 = mhc.post_pre(X, Y, H, phi2, bias2)   # this layer's post + the next layer's pre
    a    = mhc.amax(H_stack, n)                   # composite-map Amax over layers

    dX, dY, dH = mhc.post_bwd(X, Y, H, G)         # backward: G = dL/dXn
    dh = F_backward(dY)                           # the caller's sublayer backward
    dphi, dbias, dalpha = mhc.pre_bwd(X, phi, bias, dh, dH, dX, alpha=...)   # dX += ...

Tensors are torch device tensors: X [T, n, d] and h, Y [T, d] in float32 or
bfloat16; phi [n*d, n*n+2n], bias [n*n+2n] and H [T, n*n+2n] in float32.
"""
from ._binding import (EXPORTS, LIB_PATH, MAPS_HC, MAPS_MHC, MHC_BF16, MHC_FP32, OP_AMAX, OP_POST, OP_POST_BWD,
                       OP_POST_PRE, OP_PRE, OP_PRE_BWD, PRE_AUTO, PRE_ONE_PASS, PRE_ONE_PASS_FALLBACK_TEST,
                       PRE_TWO_PASS, MhcError, Params, amax, gelu_half, load_library, make_params, post, post_bwd,
                       post_bwd_workspace_size, post_pre, post_pre_ex, pre, pre_bwd, pre_bwd_workspace_size, pre_ex,
                       pre_noalloc, pre_workspace_size, workspace_size, PRE_NOALLOC_SCRATCH_BYTES)

__all__ = ["pre", "pre_ex", "pre_noalloc", "PRE_NOALLOC_SCRATCH_BYTES", "post", "post_pre", "post_pre_ex", "amax", "gelu_half", "pre_workspace_size", "post_bwd",
           "post_bwd_workspace_size", "pre_bwd", "pre_bwd_workspace_size", "workspace_size", "load_library",
           "make_params", "Params", "MhcError", "MHC_FP32", "MHC_BF16", "MAPS_MHC", "MAPS_HC", "PRE_AUTO",
           "PRE_TWO_PASS", "PRE_ONE_PASS", "PRE_ONE_PASS_FALLBACK_TEST", "OP_PRE", "OP_POST", "OP_POST_PRE",
           "OP_AMAX", "OP_POST_BWD", "OP_PRE_BWD", "LIB_PATH", "EXPORTS"]
