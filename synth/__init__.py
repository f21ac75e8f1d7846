"""Seeded synthetic inputs shared by the parity tests, the benchmark and smoke().

This module holds no arithmetic of the method.  It produces the workloads'
tensors (state X, projection phi, biases, sublayer output Y, backward seeds)
from a counter-based SplitMix64 + Box-Muller generator implemented in
``synth.c`` and records the five workload definitions.  Both the HIP path and
the oracle consume the very same bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

FP32, BF16, FP64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP for large tensors)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
        lib.synth_normal.restype = None
        _lib = lib
    return _lib


def normal(seed: int, tag: int, shape, mean: float = 0.0, std: float = 1.0, dtype: int = FP32,
           diag_n: int = 0, diag_add: float = 0.0, offset: int = 0, threads: int = 0) -> np.ndarray:
    """Normal deviates N(mean, std) (std is the standard deviation) for element
    indices [offset, offset + prod(shape)) of tensor (seed, tag).

    dtype FP32 -> float32 array, BF16 -> uint16 array of bf16 bits (RNE from
    fp32), FP64 -> float64 array."""
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    count = int(np.prod(shape)) if shape else 1
    npdt = {FP32: np.float32, BF16: np.uint16, FP64: np.float64}[dtype]
    out = np.empty(shape, dtype=npdt)
    if threads <= 0:
        threads = min(16, os.cpu_count() or 1) if count >= (1 << 20) else 1
    _load().synth_normal(seed, tag, offset, count, mean, std, dtype, diag_n, diag_add,
                         out.ctypes.data, threads)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Reinterpret bf16 bit patterns as float32 (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# Tensor tags: one independent stream per tensor of a workload.
TAG_X, TAG_PHI, TAG_BPRE, TAG_BRES, TAG_BPOST, TAG_Y, TAG_G, TAG_D = 1, 2, 3, 4, 5, 6, 7, 8


def layer_tag(layer: int, tag: int) -> int:
    """Tag of a per-layer tensor in the multi-layer stack workload."""
    return 1000 + 16 * layer + tag


@dataclass
class Workload:
    """One synthetic workload: sizes and input distributions."""
    name: str
    T: int
    n: int
    d: int
    dtype: int                  # FP32 or BF16 storage of X, h, Y, X'
    layers: int = 1
    phi_std: float = 0.02
    alpha: tuple = (0.01, 0.01, 0.01)   # alpha_pre, alpha_res, alpha_post
    b_std: float = 0.1          # b_pre, b_post
    bres_std: float = 0.1       # noise on b_res = 2 I + noise
    bres_diag: float = 2.0
    eps: float = 1e-6
    t_max: int = 20
    sublayer: str = "given"     # "given": Y drawn N(0,1); "gelu_half": Y = 0.5 GELU(h)
    maps: str = "mhc"           # "mhc": the method's maps; "hc": the unconstrained HC form (contrast)
    backward: bool = False
    seed: int = 1000
    note: str = ""

    @property
    def m(self) -> int:
        return self.n * self.n + 2 * self.n

    @property
    def K(self) -> int:
        return self.n * self.d


WORKLOADS = {
    "layer_fp32_T64_d256": Workload("layer_fp32_T64_d256", T=64, n=4, d=256, dtype=FP32, seed=1000,
                                    note="single layer forward, fp32 state"),
    "layer_bf16_T4096_d2048": Workload("layer_bf16_T4096_d2048", T=4096, n=4, d=2048, dtype=BF16, seed=1001,
                                       note="single layer forward, bf16 state, fp32 accumulation"),
    "layer_bf16_T16384_d4096": Workload("layer_bf16_T16384_d4096", T=16384, n=4, d=4096, dtype=BF16, seed=1002,
                                        note="single layer forward, bf16, batch 4 x seq 4096: headline bandwidth case"),
    "stack60_bf16_T4096_d2560": Workload("stack60_bf16_T4096_d2560", T=4096, n=4, d=2560, dtype=BF16, layers=60,
                                         bres_std=0.5, sublayer="gelu_half", seed=1003,
                                         note="60-layer stack, F = 0.5 GELU(h), composite Amax per token"),
    "layer_fwdbwd_bf16_T16384_d4096": Workload("layer_fwdbwd_bf16_T16384_d4096", T=16384, n=4, d=4096, dtype=BF16,
                                               backward=True, seed=1004,
                                               note="single layer forward + backward"),
    "hc_stack60_bf16_T4096_d2560": Workload("hc_stack60_bf16_T4096_d2560", T=4096, n=4, d=2560, dtype=BF16, layers=60,
                                            bres_diag=1.0, bres_std=0.3, sublayer="gelu_half", maps="hc", seed=1005,
                                            note="contrast: the 60-layer stack with HC's unconstrained maps, "
                                                 "b_res = I + N(0, 0.3) as in the pages' NumPy demo"),
}
WORKLOAD_ORDER = list(WORKLOADS)


def make_params(w: Workload, layer: int = 0):
    """phi [K, m] fp32, bias [m] fp32 (pre | res row-major | post) for one layer."""
    n, m, K = w.n, w.m, w.K
    tag = (lambda t: layer_tag(layer, t)) if w.layers > 1 else (lambda t: t)
    phi = normal(w.seed, tag(TAG_PHI), (K, m), 0.0, w.phi_std, FP32)
    b_pre = normal(w.seed, tag(TAG_BPRE), (n,), 0.0, w.b_std, FP32)
    b_res = normal(w.seed, tag(TAG_BRES), (n * n,), 0.0, w.bres_std, FP32, diag_n=n, diag_add=w.bres_diag)
    b_post = normal(w.seed, tag(TAG_BPOST), (n,), 0.0, w.b_std, FP32)
    bias = np.concatenate([b_pre, b_res, b_post]).astype(np.float32)
    return phi, bias


def make_state(w: Workload, T: int | None = None):
    """X [T, n, d] in the storage dtype."""
    T = w.T if T is None else T
    return normal(w.seed, TAG_X, (T, w.n, w.d), 0.0, 1.0, w.dtype)


def make_sublayer_out(w: Workload, T: int | None = None):
    """Y [T, d] in the storage dtype (the given sublayer output)."""
    T = w.T if T is None else T
    return normal(w.seed, TAG_Y, (T, w.d), 0.0, 1.0, w.dtype)


def make_grads(w: Workload, T: int | None = None):
    """G = dX_{l+1} [T, n, d] and D = dh [T, d], storage dtype."""
    T = w.T if T is None else T
    G = normal(w.seed, TAG_G, (T, w.n, w.d), 0.0, 1.0, w.dtype)
    D = normal(w.seed, TAG_D, (T, w.d), 0.0, 1.0, w.dtype)
    return G, D


def scaled(w: Workload, **changes) -> Workload:
    """Copy of a workload with some fields replaced (e.g. smaller T for tests)."""
    import dataclasses
    return dataclasses.replace(w, **changes)
