"""ctypes binding of libmhc's C ABI (include/mhc.h): argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI; this module only
turns torch tensors into device pointers, allocates outputs the caller did not
pass, and raises on a non-zero status.  There is no CPU fallback: without the
built ``libmhc.so`` the import of any entry point fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmhc.so")

MHC_FP32, MHC_BF16 = 0, 1
STATUS = {0: "MHC_OK", 1: "MHC_ERR_NULL", 2: "MHC_ERR_SHAPE", 3: "MHC_ERR_DTYPE", 4: "MHC_ERR_ALIGN",
          5: "MHC_ERR_UNSUPPORTED", 6: "MHC_ERR_ALIAS", 7: "MHC_ERR_WORKSPACE", 8: "MHC_ERR_HIP", 9: "MHC_ERR_SCRATCH"}
EXPORTS = ["mhc_pre", "mhc_pre_ex", "mhc_pre_workspace_size", "mhc_post", "mhc_amax", "mhc_gelu_half",
           "mhc_post_pre", "mhc_post_pre_ex", "mhc_post_bwd", "mhc_post_bwd_ex", "mhc_post_bwd_workspace_size", "mhc_pre_bwd", "mhc_pre_bwd_ex",
           "mhc_pre_bwd_workspace_size", "mhc_workspace_size", "mhc_pre_noalloc", "mhc_status_string",
           "mhc_abi_version"]
PRE_NOALLOC_SCRATCH_BYTES = 32 << 20
PRE_AUTO, PRE_TWO_PASS, PRE_ONE_PASS, PRE_ONE_PASS_FALLBACK_TEST = 0, 1, 2, 3
OP_PRE, OP_POST, OP_POST_PRE, OP_AMAX, OP_POST_BWD, OP_PRE_BWD = 0, 1, 2, 3, 4, 5


class MhcError(RuntimeError):
    """A libmhc entry point returned a non-zero mhc_status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


class Params(ctypes.Structure):
    """mirror of struct mhc_params"""
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("t_max", ctypes.c_int32), ("eps", ctypes.c_float),
                ("alpha_pre", ctypes.c_float), ("alpha_res", ctypes.c_float), ("alpha_post", ctypes.c_float),
                ("maps", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p


def load_library(path: str = LIB_PATH):
    """Load libmhc.so (cached).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libmhc is not built ({path} missing); run __graft_entry__.build() or "
                           f"python mhc_hyper_connections_amd/build.py")
    lib = ctypes.CDLL(path)
    lib.mhc_pre.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mhc_pre.restype = ctypes.c_int
    lib.mhc_pre_ex.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, ctypes.c_int32,
                               ctypes.POINTER(ctypes.c_int32), _P]
    lib.mhc_pre_ex.restype = ctypes.c_int
    lib.mhc_pre_workspace_size.argtypes = [ctypes.POINTER(Params)]
    lib.mhc_pre_workspace_size.restype = ctypes.c_size_t
    lib.mhc_post.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P]
    lib.mhc_post.restype = ctypes.c_int
    lib.mhc_amax.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P]
    lib.mhc_amax.restype = ctypes.c_int
    lib.mhc_gelu_half.argtypes = [ctypes.c_int64, ctypes.c_int32, _P, _P, _P]
    lib.mhc_gelu_half.restype = ctypes.c_int
    lib.mhc_post_pre.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mhc_post_pre.restype = ctypes.c_int
    lib.mhc_post_pre_ex.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), _P]
    lib.mhc_post_pre_ex.restype = ctypes.c_int
    lib.mhc_post_bwd.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P]
    lib.mhc_post_bwd.restype = ctypes.c_int
    lib.mhc_post_bwd_ex.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mhc_post_bwd_ex.restype = ctypes.c_int
    lib.mhc_post_bwd_workspace_size.argtypes = [ctypes.POINTER(Params)]
    lib.mhc_post_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mhc_pre_bwd_workspace_size.argtypes = [ctypes.POINTER(Params)]
    lib.mhc_pre_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mhc_pre_bwd.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mhc_pre_bwd.restype = ctypes.c_int
    lib.mhc_pre_bwd_ex.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                   _P]
    lib.mhc_pre_bwd_ex.restype = ctypes.c_int
    lib.mhc_pre_noalloc.argtypes = [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P]
    lib.mhc_pre_noalloc.restype = ctypes.c_int
    lib.mhc_workspace_size.argtypes = [ctypes.POINTER(Params), ctypes.c_int32]
    lib.mhc_workspace_size.restype = ctypes.c_size_t
    lib.mhc_status_string.argtypes = [ctypes.c_int]
    lib.mhc_status_string.restype = ctypes.c_char_p
    lib.mhc_abi_version.argtypes = []
    lib.mhc_abi_version.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        text = load_library().mhc_status_string(status).decode()
        raise MhcError(fn, status, text)


MAPS_MHC, MAPS_HC = 0, 1


def make_params(T, n, d, dtype, t_max=20, eps=1e-6, alpha=(0.01, 0.01, 0.01), maps=MAPS_MHC) -> Params:
    a = tuple(float(v) for v in alpha)
    return Params(int(T), int(n), int(d), int(dtype), int(t_max), float(eps), a[0], a[1], a[2], int(maps))


# ---- torch front end ---------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MHC_FP32
    if t.dtype == torch.bfloat16:
        return MHC_BF16
    raise TypeError(f"state tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libmhc works on device tensors only; move the tensors to the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("libmhc expects contiguous tensors")


def workspace_size(op, T, n, d, dtype=MHC_BF16) -> int:
    """mhc_workspace_size: scratch bytes entry point ``op`` (OP_*) needs (0: none)."""
    p = make_params(T, n, d, dtype)
    return int(load_library().mhc_workspace_size(ctypes.byref(p), int(op)))


def pre_workspace_size(T, n, d, dtype=MHC_BF16) -> int:
    p = make_params(T, n, d, dtype)
    return int(load_library().mhc_pre_workspace_size(ctypes.byref(p)))


def pre(X, phi, bias, alpha=(0.01, 0.01, 0.01), eps=1e-6, t_max=20, h=None, H=None, workspace=None,
        stream=None, algo=None, maps=MAPS_MHC):
    """mhc_pre: returns (h [T, d] state dtype, H [T, m] fp32).  With ``algo``
    (PRE_AUTO / PRE_TWO_PASS / PRE_ONE_PASS / PRE_ONE_PASS_FALLBACK_TEST) it
    calls mhc_pre_ex instead.
    ``maps``: MAPS_MHC (the method) or MAPS_HC (the unconstrained contrast)."""
    if algo is not None:
        h, H, _ = pre_ex(X, phi, bias, algo, alpha, eps, t_max, h, H, workspace, stream, maps=maps)
        return h, H
    torch = _torch()
    T, n, d = X.shape
    m = n * n + 2 * n
    p = make_params(T, n, d, _dtype_code(X), t_max, eps, alpha, maps)
    lib = load_library()
    if h is None:
        h = torch.empty((T, d), dtype=X.dtype, device=X.device)
    if H is None:
        H = torch.empty((T, m), dtype=torch.float32, device=X.device)
    need = int(lib.mhc_pre_workspace_size(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    _need_device(X, phi, bias, h, H, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mhc_pre", lib.mhc_pre(ctypes.byref(p), _ptr(X), _ptr(phi), _ptr(bias), _ptr(h), _ptr(H),
                                  _ptr(workspace), ws_bytes, _stream(stream, X.device)))
    return h, H


def pre_ex(X, phi, bias, algo=PRE_AUTO, alpha=(0.01, 0.01, 0.01), eps=1e-6, t_max=20, h=None, H=None,
           workspace=None, stream=None, maps=MAPS_MHC):
    """mhc_pre_ex: returns (h, H, algorithm that ran)."""
    torch = _torch()
    T, n, d = X.shape
    m = n * n + 2 * n
    p = make_params(T, n, d, _dtype_code(X), t_max, eps, alpha, maps)
    lib = load_library()
    if h is None:
        h = torch.empty((T, d), dtype=X.dtype, device=X.device)
    if H is None:
        H = torch.empty((T, m), dtype=torch.float32, device=X.device)
    need = int(lib.mhc_pre_workspace_size(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    _need_device(X, phi, bias, h, H, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    used = ctypes.c_int32(-1)
    _check("mhc_pre_ex", lib.mhc_pre_ex(ctypes.byref(p), _ptr(X), _ptr(phi), _ptr(bias), _ptr(h), _ptr(H),
                                        _ptr(workspace), ws_bytes, int(algo), ctypes.byref(used),
                                        _stream(stream, X.device)))
    return h, H, int(used.value)


def pre_noalloc(X, phi, bias, alpha=(0.01, 0.01, 0.01), eps=1e-6, t_max=20, h=None, H=None, stream=None,
                maps=MAPS_MHC):
    """mhc_pre_noalloc: mhc_pre on the library's static per-GPU scratch (no
    workspace).  Returns (h, H); outputs not passed are allocated here."""
    torch = _torch()
    T, n, d = X.shape
    m = n * n + 2 * n
    p = make_params(T, n, d, _dtype_code(X), t_max, eps, alpha, maps)
    if h is None:
        h = torch.empty((T, d), dtype=X.dtype, device=X.device)
    if H is None:
        H = torch.empty((T, m), dtype=torch.float32, device=X.device)
    _need_device(X, phi, bias, h, H)
    _check("mhc_pre_noalloc", load_library().mhc_pre_noalloc(ctypes.byref(p), _ptr(X), _ptr(phi), _ptr(bias),
                                                             _ptr(h), _ptr(H), _stream(stream, X.device)))
    return h, H


def post(X, Y, H, out=None, stream=None):
    """mhc_post: returns X_out [T, n, d] (``out`` may be X itself)."""
    torch = _torch()
    T, n, d = X.shape
    p = make_params(T, n, d, _dtype_code(X))
    if out is None:
        out = torch.empty_like(X)
    _need_device(X, Y, H, out)
    lib = load_library()
    _check("mhc_post", lib.mhc_post(ctypes.byref(p), _ptr(X), _ptr(Y), _ptr(H), _ptr(out),
                                    _stream(stream, X.device)))
    return out


def amax(H_stack, n, out_amax=None, gain_fwd=None, gain_bwd=None, composite=None, want_all=True, stream=None):
    """mhc_amax over H_stack [L, T, m]: returns dict of the requested outputs."""
    torch = _torch()
    L, T, m = H_stack.shape
    dev = H_stack.device
    if out_amax is None:
        out_amax = torch.empty(T, dtype=torch.float32, device=dev)
    if want_all:
        gain_fwd = torch.empty(T, dtype=torch.float32, device=dev) if gain_fwd is None else gain_fwd
        gain_bwd = torch.empty(T, dtype=torch.float32, device=dev) if gain_bwd is None else gain_bwd
        composite = torch.empty((T, n, n), dtype=torch.float32, device=dev) if composite is None else composite
    _need_device(H_stack, out_amax, gain_fwd, gain_bwd, composite)
    lib = load_library()
    _check("mhc_amax", lib.mhc_amax(T, n, L, _ptr(H_stack), _ptr(out_amax), _ptr(gain_fwd), _ptr(gain_bwd),
                                    _ptr(composite), _stream(stream, dev)))
    return {"amax": out_amax, "gain_fwd": gain_fwd, "gain_bwd": gain_bwd, "composite": composite}


def gelu_half(h, out=None, stream=None):
    """The stack workload's sublayer: out = 0.5 GELU(h), state dtype."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(h)
    _need_device(h, out)
    lib = load_library()
    _check("mhc_gelu_half", lib.mhc_gelu_half(h.numel(), _dtype_code(h), _ptr(h), _ptr(out),
                                              _stream(stream, h.device)))
    return out


def post_bwd_workspace_size(T, n, d, dtype=MHC_BF16) -> int:
    """Bytes of workspace that lets mhc_post_bwd_ex take its tiled form (0: none)."""
    return int(load_library().mhc_post_bwd_workspace_size(ctypes.byref(make_params(T, n, d, dtype))))


def post_bwd(X, Y, H, G, dX=None, dY=None, dH=None, workspace=None, tiled=True, stream=None, skip_dX=False):
    """mhc_post_bwd_ex: returns (dX [T, n, d], dY [T, d], dH [T, m]); dH's first
    n columns (the read map's) are left as they were.  With ``tiled`` (and d a
    multiple of 512) the call runs the tiled form, on ``workspace`` or on a
    buffer allocated here; ``tiled=False`` runs mhc_post_bwd, which needs none.
    ``skip_dX``: dX is not written (passed as NULL; returned as None), for
    pre_bwd(..., G=G), which then forms the whole dX."""
    torch = _torch()
    T, n, d = X.shape
    m = n * n + 2 * n
    p = make_params(T, n, d, _dtype_code(X))
    if skip_dX:
        dX = None
    elif dX is None:
        dX = torch.empty_like(X)
    dY = torch.empty_like(Y) if dY is None else dY
    dH = torch.zeros((T, m), dtype=torch.float32, device=X.device) if dH is None else dH
    _need_device(X, Y, H, G, dY, dH)
    if dX is not None:
        _need_device(dX)
    lib = load_library()
    if not tiled:
        _check("mhc_post_bwd", lib.mhc_post_bwd(ctypes.byref(p), _ptr(X), _ptr(Y), _ptr(H), _ptr(G), _ptr(dX),
                                                _ptr(dY), _ptr(dH), _stream(stream, X.device)))
        return dX, dY, dH
    need = int(lib.mhc_post_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_bytes = 0
    if workspace is not None:
        _need_device(workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("mhc_post_bwd_ex", lib.mhc_post_bwd_ex(ctypes.byref(p), _ptr(X), _ptr(Y), _ptr(H), _ptr(G), _ptr(dX),
                                                  _ptr(dY), _ptr(dH), _ptr(workspace),
                                                  ws_bytes, _stream(stream, X.device)))
    return dX, dY, dH


def pre_bwd_workspace_size(T, n, d, dtype=MHC_BF16) -> int:
    p = make_params(T, n, d, dtype)
    return int(load_library().mhc_pre_bwd_workspace_size(ctypes.byref(p)))


def pre_bwd(X, phi, bias, D, dH, dX, alpha=(0.01, 0.01, 0.01), eps=1e-6, t_max=20, dphi=None, dbias=None,
            dalpha=None, workspace=None, stream=None, G=None):
    """mhc_pre_bwd: adds the read map's and the maps' share to dX (in place)
    and returns (dphi [n*d, m], dbias [m], dalpha [3]), all fp32.  With G
    (dL/dX_out) it calls mhc_pre_bwd_ex, which writes the whole dX (after
    post_bwd(..., skip_dX=True))."""
    torch = _torch()
    T, n, d = X.shape
    m = n * n + 2 * n
    p = make_params(T, n, d, _dtype_code(X), t_max, eps, alpha)
    lib = load_library()
    dev = X.device
    dphi = torch.empty((n * d, m), dtype=torch.float32, device=dev) if dphi is None else dphi
    dbias = torch.empty(m, dtype=torch.float32, device=dev) if dbias is None else dbias
    dalpha = torch.empty(3, dtype=torch.float32, device=dev) if dalpha is None else dalpha
    need = int(lib.mhc_pre_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need_device(X, phi, bias, D, dH, dX, dphi, dbias, dalpha, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    if G is None:
        _check("mhc_pre_bwd", lib.mhc_pre_bwd(ctypes.byref(p), _ptr(X), _ptr(phi), _ptr(bias), _ptr(D), _ptr(dH),
                                              _ptr(dX), _ptr(dphi), _ptr(dbias), _ptr(dalpha), _ptr(workspace),
                                              ws_bytes, _stream(stream, dev)))
    else:
        _need_device(G)
        _check("mhc_pre_bwd_ex", lib.mhc_pre_bwd_ex(ctypes.byref(p), _ptr(X), _ptr(phi), _ptr(bias), _ptr(D),
                                                    _ptr(dH), _ptr(G), _ptr(dX), _ptr(dphi), _ptr(dbias),
                                                    _ptr(dalpha), _ptr(workspace), ws_bytes, _stream(stream, dev)))
    return dphi, dbias, dalpha


def post_pre(X, Y, H, phi, bias, alpha=(0.01, 0.01, 0.01), eps=1e-6, t_max=20, out=None, h=None, H_next=None,
             workspace=None, stream=None, maps=MAPS_MHC):
    """mhc_post_pre: layer l's mixing, then layer l+1's maps and sublayer
    input.  Returns (X_next [T, n, d], h [T, d], H_next [T, m]); ``out`` may
    be X itself."""
    X_next, h, H_next, _ = post_pre_ex(X, Y, H, phi, bias, PRE_AUTO, alpha=alpha, eps=eps, t_max=t_max, out=out, h=h,
                                       H_next=H_next, workspace=workspace, stream=stream, maps=maps)
    return X_next, h, H_next


def post_pre_ex(X, Y, H, phi, bias, algo=PRE_AUTO, alpha=(0.01, 0.01, 0.01), eps=1e-6, t_max=20, out=None, h=None,
                H_next=None, workspace=None, stream=None, maps=MAPS_MHC):
    """mhc_post_pre_ex: returns (X_next, h, H_next, algorithm that ran)."""
    torch = _torch()
    T, n, d = X.shape
    m = n * n + 2 * n
    p = make_params(T, n, d, _dtype_code(X), t_max, eps, alpha, maps)
    lib = load_library()
    out = torch.empty_like(X) if out is None else out
    h = torch.empty((T, d), dtype=X.dtype, device=X.device) if h is None else h
    H_next = torch.empty((T, m), dtype=torch.float32, device=X.device) if H_next is None else H_next
    need = int(lib.mhc_pre_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=X.device)
    _need_device(X, Y, H, phi, bias, out, h, H_next, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    used = ctypes.c_int32(-1)
    _check("mhc_post_pre_ex", lib.mhc_post_pre_ex(ctypes.byref(p), _ptr(X), _ptr(Y), _ptr(H), _ptr(out), _ptr(phi),
                                                  _ptr(bias), _ptr(h), _ptr(H_next), _ptr(workspace), ws_bytes,
                                                  int(algo), ctypes.byref(used), _stream(stream, X.device)))
    return out, h, H_next, int(used.value)
