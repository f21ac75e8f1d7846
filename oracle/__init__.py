"""CPU oracle of the mHC layer: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``mhc_oracle.cpp`` (plain,
single-threaded C++ in double precision, built with ``g++ -O2`` and no
fast-math) through ctypes and shares no code with the HIP library.

Every function takes numpy arrays: the state in its storage form (float32, or
uint16 bf16 bit patterns), parameters in float32, and returns float64 results
for the listed tokens.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhc_oracle.cpp")
_LIB = os.path.join(_HERE, "libmhc_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_D = ctypes.c_double


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle (g++ -O2, no fast-math).  ``src``/``out`` let the
    planted-mistake tests build altered copies under a temporary directory."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fno-fast-math",
                               "-o", tmp, src])
        os.replace(tmp, out)
    return out


def _bind(lib):
    lib.mhcref_version.restype = _I32
    lib.mhcref_round_bf16.argtypes = [_P, _P, _I64]
    lib.mhcref_round_bf16.restype = None
    lib.mhcref_sinkhorn.argtypes = [_I32, _P, _I32, _P, _P]
    lib.mhcref_sinkhorn.restype = None
    lib.mhcref_pre.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _D, _I32, _P, _I64,
                               _P, _P, _P, _P, _P, _P]
    lib.mhcref_pre.restype = _I32
    lib.mhcref_post.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _I64, _P]
    lib.mhcref_post.restype = _I32
    for name in ("mhcref_amax", "mhcref_amax_f64"):
        f = getattr(lib, name)
        f.argtypes = [_I64, _I32, _I32, _P, _P, _I64, _P, _P, _P, _P]
        f.restype = _I32
    lib.mhcref_gelu_half.argtypes = [_I64, _I32, _P, _P]
    lib.mhcref_gelu_half.restype = _I32
    lib.mhcref_stack.argtypes = [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _D, _I32, _P, _I64,
                                 _P, _P, _P, _P, _P, _P]
    lib.mhcref_stack.restype = _I32
    lib.mhcref_pre_hc.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _D, _P, _I64, _P, _P]
    lib.mhcref_pre_hc.restype = _I32
    lib.mhcref_stack_hc.argtypes = [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _D, _P, _I64,
                                    _P, _P, _P, _P, _P]
    lib.mhcref_stack_hc.restype = _I32
    lib.mhcref_bwd.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _D, _I32, _P, _P, _P, _I64,
                               _P, _P, _P, _P, _P, _P, _P]
    lib.mhcref_bwd.restype = _I32
    lib.mhcref_layer_f64.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P, _D, _I32, _P, _P]
    lib.mhcref_layer_f64.restype = _I32
    lib.mhcref_bwd_f64.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P, _D, _I32, _P, _P,
                                   _P, _P, _P, _P, _P, _P, _P]
    lib.mhcref_bwd_f64.restype = _I32
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it if it is absent).  With ``path``
    a separately built copy is loaded and returned without caching."""
    global _lib
    if path is not None:
        return Oracle(_bind(ctypes.CDLL(path)))
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = Oracle(_bind(ctypes.CDLL(_LIB)))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(X: np.ndarray) -> int:
    if X.dtype == np.float32:
        return 0
    if X.dtype == np.uint16:
        return 1
    raise TypeError("state must be float32 or uint16 (bf16 bits)")


def _tokens(T, tokens):
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))


class Oracle:
    """Thin numpy front end of one loaded oracle library."""

    def __init__(self, lib):
        self.lib = lib

    def round_bf16(self, v) -> np.ndarray:
        v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.mhcref_round_bf16(_ptr(v), _ptr(out), v.size)
        return out

    def sinkhorn(self, logits, t_max: int = 20, trace: bool = False):
        """Sinkhorn-Knopp on exp(logits) (n x n).  With trace=True also returns
        an array [t_max, 2 (after col step / after row step), 2 (row sums / col sums), n]."""
        L = np.ascontiguousarray(np.asarray(logits, dtype=np.float64))
        n = L.shape[0]
        assert L.shape == (n, n)
        out = np.empty((n, n), dtype=np.float64)
        tr = np.empty((t_max, 2, 2, n), dtype=np.float64) if trace else None
        self.lib.mhcref_sinkhorn(n, _ptr(L), t_max, _ptr(out), _ptr(tr))
        return (out, tr) if trace else out

    def pre(self, X, phi, bias, alpha, eps=1e-6, t_max=20, tokens=None, want_h=True, extras=False):
        """Maps and aggregation.  X [T, n, d]; returns dict with H [ntok, m],
        h [ntok, d] and, with extras, r, z, logit, sk_err."""
        X = np.ascontiguousarray(X)
        T, n, d = X.shape
        m = n * n + 2 * n
        phi = np.ascontiguousarray(phi, dtype=np.float32)
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert phi.shape == (n * d, m) and bias.shape == (m,)
        a3 = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32).reshape(3))
        tok = _tokens(T, tokens)
        q = tok.size
        H = np.empty((q, m))
        h = np.empty((q, d)) if want_h else None
        r = np.empty(q) if extras else None
        z = np.empty((q, m)) if extras else None
        lg = np.empty((q, m)) if extras else None
        sk = np.empty((q, 4)) if extras else None
        rc = self.lib.mhcref_pre(T, n, d, _dtype_code(X), _ptr(X), _ptr(phi), _ptr(bias), _ptr(a3),
                                 float(eps), int(t_max), _ptr(tok), q, _ptr(h), _ptr(H), _ptr(r),
                                 _ptr(z), _ptr(lg), _ptr(sk))
        if rc != 0:
            raise ValueError(f"mhcref_pre rejected its arguments ({rc})")
        out = {"H": H, "h": h}
        if extras:
            out.update(r=r, z=z, logit=lg, sk_err=sk)
        return out

    def post(self, X, Y, H_rows, tokens=None):
        """X' for the listed tokens.  H_rows [ntok, m] fp32 (row q for tokens[q])."""
        X = np.ascontiguousarray(X)
        Y = np.ascontiguousarray(Y)
        T, n, d = X.shape
        assert Y.shape == (T, d) and Y.dtype == X.dtype
        tok = _tokens(T, tokens)
        Hc = np.ascontiguousarray(H_rows, dtype=np.float32)
        assert Hc.shape == (tok.size, n * n + 2 * n)
        out = np.empty((tok.size, n, d))
        rc = self.lib.mhcref_post(T, n, d, _dtype_code(X), _ptr(X), _ptr(Y), _ptr(Hc), _ptr(tok),
                                  tok.size, _ptr(out))
        if rc != 0:
            raise ValueError(f"mhcref_post rejected its arguments ({rc})")
        return out

    def amax(self, H_stack, n: int, tokens=None):
        """Composite Amax.  H_stack [L, T, m] (float32 or float64).  Returns
        dict amax, gain_fwd, gain_bwd [ntok] and composite [ntok, n, n]."""
        Hs = np.ascontiguousarray(H_stack)
        L, T, m = Hs.shape
        assert m == n * n + 2 * n
        tok = _tokens(T, tokens)
        q = tok.size
        a, f, b, c = np.empty(q), np.empty(q), np.empty(q), np.empty((q, n, n))
        fn = self.lib.mhcref_amax_f64 if Hs.dtype == np.float64 else self.lib.mhcref_amax
        if Hs.dtype not in (np.float64, np.float32):
            raise TypeError("H_stack must be float32 or float64")
        rc = fn(T, n, L, _ptr(Hs), _ptr(tok), q, _ptr(a), _ptr(f), _ptr(b), _ptr(c))
        if rc != 0:
            raise ValueError(f"mhcref_amax rejected its arguments ({rc})")
        return {"amax": a, "gain_fwd": f, "gain_bwd": b, "composite": c}

    def gelu_half(self, h):
        h = np.ascontiguousarray(h)
        y = np.empty(h.shape)
        code = 0 if h.dtype == np.float32 else 1
        assert h.dtype in (np.float32, np.uint16)
        rc = self.lib.mhcref_gelu_half(h.size, code, _ptr(h), _ptr(y))
        assert rc == 0
        return y

    def stack(self, X0, phis, biases, alphas, eps=1e-6, t_max=20, tokens=None, want_sk=False):
        """L-layer stack with F = 0.5 GELU.  Returns dict X (storage dtype
        [ntok, n, d]), H [L, ntok, m] fp32, amax, gain_fwd, gain_bwd [ntok]."""
        X0 = np.ascontiguousarray(X0)
        T, n, d = X0.shape
        m = n * n + 2 * n
        phis = np.ascontiguousarray(phis, dtype=np.float32)
        L = phis.shape[0]
        assert phis.shape == (L, n * d, m)
        biases = np.ascontiguousarray(biases, dtype=np.float32)
        alphas = np.ascontiguousarray(alphas, dtype=np.float32)
        assert biases.shape == (L, m) and alphas.shape == (L, 3)
        tok = _tokens(T, tokens)
        q = tok.size
        Xf = np.empty((q, n, d), dtype=X0.dtype)
        Hs = np.empty((L, q, m), dtype=np.float32)
        a, f, b = np.empty(q), np.empty(q), np.empty(q)
        sk = np.empty((L, q, 4)) if want_sk else None
        rc = self.lib.mhcref_stack(T, n, d, _dtype_code(X0), L, _ptr(X0), _ptr(phis), _ptr(biases),
                                   _ptr(alphas), float(eps), int(t_max), _ptr(tok), q, _ptr(Xf),
                                   _ptr(Hs), _ptr(a), _ptr(f), _ptr(b), _ptr(sk))
        if rc != 0:
            raise ValueError(f"mhcref_stack rejected its arguments ({rc})")
        out = {"X": Xf, "H": Hs, "amax": a, "gain_fwd": f, "gain_bwd": b}
        if want_sk:
            out["sk_err"] = sk
        return out

    def bwd(self, X, Y, phi, bias, alpha, G, D, eps=1e-6, t_max=20, tokens=None):
        """Gradients of sum_t <G_t, X'_t> + <D_t, h_t> for the listed tokens.
        X, G [T, n, d] and Y, D [T, d] in the storage form.  Returns dict dX
        [ntok, n, d], dY [ntok, d], dH, dlogit [ntok, m] and dphi [n*d, m],
        dbias [m], dalpha [3] summed over the listed tokens (all float64)."""
        X, Y, G, D = (np.ascontiguousarray(a) for a in (X, Y, G, D))
        T, n, d = X.shape
        m = n * n + 2 * n
        assert G.shape == X.shape and Y.shape == (T, d) and D.shape == (T, d)
        assert X.dtype == Y.dtype == G.dtype == D.dtype
        phi = np.ascontiguousarray(phi, dtype=np.float32)
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        a3 = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32).reshape(3))
        tok = _tokens(T, tokens)
        q = tok.size
        out = {"dX": np.empty((q, n, d)), "dY": np.empty((q, d)), "dH": np.empty((q, m)),
               "dlogit": np.empty((q, m)), "dphi": np.empty((n * d, m)), "dbias": np.empty(m),
               "dalpha": np.empty(3)}
        rc = self.lib.mhcref_bwd(T, n, d, _dtype_code(X), _ptr(X), _ptr(Y), _ptr(phi), _ptr(bias), _ptr(a3),
                                 float(eps), int(t_max), _ptr(G), _ptr(D), _ptr(tok), q, _ptr(out["dX"]),
                                 _ptr(out["dY"]), _ptr(out["dH"]), _ptr(out["dlogit"]), _ptr(out["dphi"]),
                                 _ptr(out["dbias"]), _ptr(out["dalpha"]))
        if rc != 0:
            raise ValueError(f"mhcref_bwd rejected its arguments ({rc})")
        return out

    @staticmethod
    def _f64(*arrays):
        return [np.ascontiguousarray(a, dtype=np.float64) for a in arrays]

    def layer_f64(self, X, Y, phi, bias, alpha, eps=1e-6, t_max=20):
        """The layer forward with every value in double: returns (h [T, d], X' [T, n, d])."""
        X, Y, phi, bias, alpha = self._f64(X, Y, phi, bias, np.asarray(alpha).reshape(3))
        T, n, d = X.shape
        h, Xo = np.empty((T, d)), np.empty((T, n, d))
        rc = self.lib.mhcref_layer_f64(T, n, d, _ptr(X), _ptr(Y), _ptr(phi), _ptr(bias), _ptr(alpha), float(eps),
                                       int(t_max), _ptr(h), _ptr(Xo))
        if rc != 0:
            raise ValueError(f"mhcref_layer_f64 rejected its arguments ({rc})")
        return h, Xo

    def bwd_f64(self, X, Y, phi, bias, alpha, G, D, eps=1e-6, t_max=20):
        """Backward of layer_f64 over all tokens; same dict as bwd."""
        X, Y, phi, bias, alpha, G, D = self._f64(X, Y, phi, bias, np.asarray(alpha).reshape(3), G, D)
        T, n, d = X.shape
        m = n * n + 2 * n
        out = {"dX": np.empty((T, n, d)), "dY": np.empty((T, d)), "dH": np.empty((T, m)),
               "dlogit": np.empty((T, m)), "dphi": np.empty((n * d, m)), "dbias": np.empty(m),
               "dalpha": np.empty(3)}
        rc = self.lib.mhcref_bwd_f64(T, n, d, _ptr(X), _ptr(Y), _ptr(phi), _ptr(bias), _ptr(alpha), float(eps),
                                     int(t_max), _ptr(G), _ptr(D), _ptr(out["dX"]), _ptr(out["dY"]),
                                     _ptr(out["dH"]), _ptr(out["dlogit"]), _ptr(out["dphi"]), _ptr(out["dbias"]),
                                     _ptr(out["dalpha"]))
        if rc != 0:
            raise ValueError(f"mhcref_bwd_f64 rejected its arguments ({rc})")
        return out

    def pre_hc(self, X, phi, bias, alpha, eps=1e-6, tokens=None):
        """HC-form maps (bias + alpha * tanh(z)) and aggregation: dict H, h."""
        X = np.ascontiguousarray(X)
        T, n, d = X.shape
        m = n * n + 2 * n
        phi = np.ascontiguousarray(phi, dtype=np.float32)
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        a3 = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32).reshape(3))
        tok = _tokens(T, tokens)
        q = tok.size
        H, h = np.empty((q, m)), np.empty((q, d))
        rc = self.lib.mhcref_pre_hc(T, n, d, _dtype_code(X), _ptr(X), _ptr(phi), _ptr(bias), _ptr(a3), float(eps),
                                    _ptr(tok), q, _ptr(h), _ptr(H))
        if rc != 0:
            raise ValueError(f"mhcref_pre_hc rejected its arguments ({rc})")
        return {"H": H, "h": h}

    def stack_hc(self, X0, phis, biases, alphas, eps=1e-6, tokens=None):
        """The L-layer stack with HC-form maps; same outputs as stack()."""
        X0 = np.ascontiguousarray(X0)
        T, n, d = X0.shape
        m = n * n + 2 * n
        phis = np.ascontiguousarray(phis, dtype=np.float32)
        L = phis.shape[0]
        biases = np.ascontiguousarray(biases, dtype=np.float32)
        alphas = np.ascontiguousarray(alphas, dtype=np.float32)
        tok = _tokens(T, tokens)
        q = tok.size
        Xf = np.empty((q, n, d), dtype=X0.dtype)
        Hs = np.empty((L, q, m), dtype=np.float32)
        a, f, b = np.empty(q), np.empty(q), np.empty(q)
        rc = self.lib.mhcref_stack_hc(T, n, d, _dtype_code(X0), L, _ptr(X0), _ptr(phis), _ptr(biases), _ptr(alphas),
                                      float(eps), _ptr(tok), q, _ptr(Xf), _ptr(Hs), _ptr(a), _ptr(f), _ptr(b))
        if rc != 0:
            raise ValueError(f"mhcref_stack_hc rejected its arguments ({rc})")
        return {"X": Xf, "H": Hs, "amax": a, "gain_fwd": f, "gain_bwd": b}
