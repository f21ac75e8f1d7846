"""The C-ABI library on the host: it loads, exports every declared symbol and
rejects bad arguments before anything reaches a device.  No GPU needed: all
calls here return from the host-side checks."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")


@pytest.fixture(scope="module")
def lib():
    import mhc_hyper_connections_amd as m
    # tests/test_sanitizers.py runs these checks again on a copy of the
    # library whose host code is built with AddressSanitizer and
    # UndefinedBehaviorSanitizer, named here.
    san = os.environ.get("MHC_TEST_LIBMHC")
    if san:
        return m.load_library(san)
    if not os.path.exists(m.LIB_PATH):
        from mhc_hyper_connections_amd import build
        build.build(force=False)
    return m.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"mhc_pre", "mhc_post", "mhc_amax", "mhc_pre_workspace_size"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/mhc.h but not exported"
    import mhc_hyper_connections_amd as m
    assert set(m.EXPORTS) == set(names)


def test_abi_version_and_status_strings(lib):
    ver = int(re.search(r"#define MHC_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.mhc_abi_version() == ver
    for s in range(10):
        assert lib.mhc_status_string(s) and lib.mhc_status_string(s) != b"unknown status"
    assert lib.mhc_status_string(12345) == b"unknown status"


def _params(**kw):
    import mhc_hyper_connections_amd as m
    base = dict(T=64, n=4, d=256, dtype=m.MHC_BF16, t_max=20, eps=1e-6, alpha=(0.01, 0.01, 0.01), maps=m.MAPS_MHC)
    base.update(kw)
    return m.make_params(**base)


# Fake, never-dereferenced device addresses, far apart and 16-byte aligned.
A = [0x10000000 * (k + 1) for k in range(8)]


def _pre(lib, p, X=A[0], phi=A[1], bias=A[2], h=A[3], H=A[4], ws=A[5], ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.mhc_pre_workspace_size(ctypes.byref(p))
    return lib.mhc_pre(ctypes.byref(p), X, phi, bias, h, H, ws, ws_bytes, None)


def test_pre_argument_checks(lib):
    assert lib.mhc_pre(None, A[0], A[1], A[2], A[3], A[4], A[5], 1 << 30, None) == 1      # NULL params
    assert _pre(lib, _params(n=3)) == 5                                                     # UNSUPPORTED
    assert _pre(lib, _params(n=0)) == 2                                                     # SHAPE
    assert _pre(lib, _params(d=12)) == 5                                                    # d % 8
    assert _pre(lib, _params(dtype=7)) == 3                                                 # DTYPE
    assert _pre(lib, _params(T=-1)) == 2
    assert _pre(lib, _params(t_max=-1)) == 2
    assert _pre(lib, _params(eps=float("nan"))) == 2
    assert _pre(lib, _params(eps=-1.0)) == 2
    assert _pre(lib, _params(alpha=(float("inf"), 0, 0))) == 2
    assert _pre(lib, _params(), X=None) == 1
    assert _pre(lib, _params(), H=None) == 1
    assert _pre(lib, _params(), X=A[0] + 8) == 4                                            # ALIGN
    assert _pre(lib, _params(), ws=None) == 7                                               # WORKSPACE
    p = _params()
    need = lib.mhc_pre_workspace_size(ctypes.byref(p))
    assert _pre(lib, p, ws_bytes=need - 1) == 7
    assert _pre(lib, _params(), h=A[0] + 16) == 6                                           # h inside X
    assert _pre(lib, _params(), H=A[3]) == 6                                                # H on h
    assert _pre(lib, _params(), ws=A[4]) == 6                                               # ws on H
    assert _pre(lib, _params(T=0), X=None, phi=None) == 0                                   # no-op


def test_pre_ex_argument_checks(lib):
    p = _params()
    need = lib.mhc_pre_workspace_size(ctypes.byref(p))
    used = ctypes.c_int32(-1)
    assert lib.mhc_pre_ex(ctypes.byref(p), A[0], A[1], A[2], A[3], A[4], A[5], need, 7, ctypes.byref(used), None) == 2
    assert used.value == 1                                  # reported even when refused
    assert lib.mhc_pre_ex(ctypes.byref(_params(n=3)), A[0], A[1], A[2], A[3], A[4], A[5], need, 2, None, None) == 5
    assert lib.mhc_pre_ex(ctypes.byref(_params(T=0)), None, None, None, None, None, None, 0, 2, None, None) == 0


def test_workspace_size_formula(lib):
    # [256-byte header, which only the single pass uses][body: the largest of the forms' records]
    for (T, n, d) in ((64, 4, 256), (16384, 4, 4096), (5, 2, 264), (1, 1, 8), (4096, 4, 2560)):
        p = _params(T=T, n=n, d=d)
        slices = -(-d // 256)
        width = ((n * n + 2 * n + 1) & ~1) + 2          # m fp32 partials, then an aligned fp64
        body = slices * T * width * 4 + 512 * 16        # records + write-only trash slots (16 B per thread)
        if -(-T // 32) * slices < 128:                  # small-T form: slices of 64 positions
            body = max(body, -(-d // 64) * T * width * 4 + 512 * 16)
        # one pass: 16 start words per team, then per team 5 ring slots of 16-token
        # records (m + 2 words per member and token) and n H_pre words per token, 8 B a word;
        # room for 8 XCDs x floor(48 / slices) teams
        teams = 8 * (48 // slices)
        record = ((n * n + 2 * n + 1) & ~1) + 2            # m partials, even padding, fp64 sum of squares
        slot = slices * 16 * record + 16 * n
        one_pass = teams * 16 * 8 + teams * 5 * slot * 8 if 8 <= slices <= 16 else 0
        assert lib.mhc_pre_workspace_size(ctypes.byref(p)) == 256 + max(body, one_pass)
    for (T, d) in ((64, 256), (1, 8), (4096, 4104)):
        # n = 8: records of 80 partials, 2 words of padding and an fp64 (84 words, 16-byte
        # aligned) over slices of 512 positions of one stream, plus trash slots
        p = _params(T=T, n=8, d=d)
        assert lib.mhc_pre_workspace_size(ctypes.byref(p)) == 256 + 8 * -(-d // 512) * T * 84 * 4 + 512 * 16
    assert lib.mhc_pre_workspace_size(None) == 0
    assert lib.mhc_pre_workspace_size(ctypes.byref(_params(n=3))) == 0


def test_workspace_size_query_by_op(lib):
    """mhc_workspace_size(p, op) answers for every entry point: the same
    numbers as the per-entry-point queries, 0 for those that need no scratch,
    for invalid parameters and for unknown op codes."""
    import mhc_hyper_connections_amd as m
    for (T, n, d, dt) in ((64, 4, 256, 0), (16384, 4, 4096, 1), (5, 2, 264, 1), (100, 8, 512, 1), (33, 1, 1024, 0)):
        p = _params(T=T, n=n, d=d, dtype=dt)
        q = ctypes.byref(p)
        assert lib.mhc_workspace_size(q, m.OP_PRE) == lib.mhc_pre_workspace_size(q) > 0
        assert lib.mhc_workspace_size(q, m.OP_POST_PRE) == lib.mhc_pre_workspace_size(q)
        assert lib.mhc_workspace_size(q, m.OP_POST_BWD) == lib.mhc_post_bwd_workspace_size(q)
        assert lib.mhc_workspace_size(q, m.OP_PRE_BWD) == lib.mhc_pre_bwd_workspace_size(q)
        assert lib.mhc_workspace_size(q, m.OP_POST) == 0
        assert lib.mhc_workspace_size(q, m.OP_AMAX) == 0
        for bad in (-1, 6, 1000):
            assert lib.mhc_workspace_size(q, bad) == 0
    for op in range(6):
        assert lib.mhc_workspace_size(None, op) == 0
        assert lib.mhc_workspace_size(ctypes.byref(_params(n=3)), op) == 0
    assert m.workspace_size(m.OP_PRE_BWD, 16384, 4, 4096) == m.pre_bwd_workspace_size(16384, 4, 4096)


def test_post_argument_checks(lib):
    p = _params()
    post = lambda p, X=A[0], Y=A[1], H=A[2], O=A[3]: lib.mhc_post(ctypes.byref(p), X, Y, H, O, None)
    assert lib.mhc_post(None, A[0], A[1], A[2], A[3], None) == 1
    assert post(_params(n=3)) == 5
    assert post(p, Y=None) == 1
    assert post(p, O=A[3] + 4) == 4
    assert post(p, O=A[0] + 1024) == 6               # partial overlap with X
    assert post(p, O=A[1]) == 6                      # onto Y
    assert post(_params(T=0), X=None, Y=None, H=None, O=None) == 0


def test_amax_and_gelu_argument_checks(lib):
    assert lib.mhc_amax(10, 3, 5, A[0], A[1], None, None, None, None) == 5
    assert lib.mhc_amax(10, 16, 5, A[0], A[1], None, None, None, None) == 5
    assert lib.mhc_amax(10, 8, 5, A[0], A[0], None, None, None, None) == 6   # n = 8 passes the shape checks
    assert lib.mhc_amax(-1, 4, 5, A[0], A[1], None, None, None, None) == 2
    assert lib.mhc_amax(10, 4, -1, A[0], A[1], None, None, None, None) == 2
    assert lib.mhc_amax(10, 4, 5, None, A[1], None, None, None, None) == 1
    assert lib.mhc_amax(10, 4, 5, A[0], None, None, None, None, None) == 1
    assert lib.mhc_amax(10, 4, 5, A[0], A[0], None, None, None, None) == 6
    assert lib.mhc_amax(10, 4, 5, A[0], A[1], A[1], None, None, None) == 6
    assert lib.mhc_amax(0, 4, 5, None, None, None, None, None, None) == 0
    assert lib.mhc_gelu_half(10, 9, A[0], A[1], None) == 3
    assert lib.mhc_gelu_half(-1, 1, A[0], A[1], None) == 2
    assert lib.mhc_gelu_half(10, 1, A[0] + 2, A[1], None) == 4
    assert lib.mhc_gelu_half(100, 1, A[0], A[0] + 16, None) == 6


def test_binding_refuses_host_tensors_and_missing_library(lib):
    torch = pytest.importorskip("torch")
    import mhc_hyper_connections_amd as m
    X = torch.zeros((4, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m.post(X, torch.zeros((4, 64), dtype=torch.bfloat16), torch.zeros((4, 24)))
    with pytest.raises(RuntimeError, match="not built"):
        m.load_library("/nonexistent/libmhc.so")


def test_post_bwd_argument_checks(lib):
    p = _params()
    f = lambda p, X=A[0], Y=A[1], H=A[2], G=A[3], dX=A[4], dY=A[5], dH=A[6]: \
        lib.mhc_post_bwd(ctypes.byref(p), X, Y, H, G, dX, dY, dH, None)
    assert lib.mhc_post_bwd(None, *A[:7], None) == 1
    assert f(_params(n=3)) == 5
    assert f(_params(n=8)) == 5                        # the backward covers n <= 4
    assert f(p, G=None) == 1
    assert f(p, dH=A[6] + 4) == 4
    assert f(p, dX=A[3]) == 6                         # dX onto G
    assert f(p, dY=A[4] + 64) == 6                    # dY inside dX
    assert f(p, dH=A[0]) == 6                         # dH onto X
    assert f(_params(T=0), X=None, Y=None, H=None, G=None, dX=None, dY=None, dH=None) == 0


def test_post_bwd_ex_workspace(lib):
    """The tiled form's workspace: T x (d / 512) slices x (n*n + n) floats,
    0 where d is not a multiple of 512; a short, misaligned or overlapping
    workspace is refused."""
    for T, n, d in ((64, 4, 512), (1000, 4, 4096), (7, 2, 1024), (3, 1, 1536)):
        assert lib.mhc_post_bwd_workspace_size(ctypes.byref(_params(T=T, n=n, d=d))) == T * (d // 512) * (n * n + n) * 4
    for d in (256, 520, 1000):
        assert lib.mhc_post_bwd_workspace_size(ctypes.byref(_params(d=d))) == 0
    assert lib.mhc_post_bwd_workspace_size(ctypes.byref(_params(n=8, d=512))) == 0
    assert lib.mhc_post_bwd_workspace_size(None) == 0
    p = _params(d=512)
    need = lib.mhc_post_bwd_workspace_size(ctypes.byref(p))
    f = lambda p, ws=A[7], nb=need, dX=A[4]: \
        lib.mhc_post_bwd_ex(ctypes.byref(p), A[0], A[1], A[2], A[3], dX, A[5], A[6], ws, nb, None)
    assert f(p, nb=need - 1) == 7                     # WORKSPACE
    assert f(p, ws=A[7] + 8) == 4                     # ALIGN
    assert f(p, ws=A[4] + 64) == 6                    # workspace inside dX
    assert f(_params(n=8, d=512)) == 5


def test_pre_bwd_argument_checks(lib):
    p = _params()
    need = lib.mhc_pre_bwd_workspace_size(ctypes.byref(p))
    assert need > 0

    def f(p, X=A[0], phi=A[1], bias=A[2], D=A[3], dH=A[4], dX=A[5], dphi=A[6], dbias=A[7],
          dalpha=A[7] + 4096, ws=A[7] + 8192, ws_bytes=None):
        nb = lib.mhc_pre_bwd_workspace_size(ctypes.byref(p)) if ws_bytes is None else ws_bytes
        return lib.mhc_pre_bwd(ctypes.byref(p), X, phi, bias, D, dH, dX, dphi, dbias, dalpha, ws, nb, None)
    assert f(_params(n=3)) == 5
    assert f(_params(n=8)) == 5                        # the backward covers n <= 4
    assert lib.mhc_pre_bwd_workspace_size(ctypes.byref(_params(n=8))) == 0
    assert f(_params(t_max=129)) == 5                  # Sinkhorn iterates beyond the backward's LDS budget
    assert f(p, D=None) == 1
    assert f(p, ws=None) == 7
    assert f(p, ws_bytes=need - 1) == 7
    assert f(p, dphi=A[6] + 8) == 4
    assert f(p, dX=A[0]) == 6                          # dX onto X
    assert f(p, dbias=A[6]) == 6                       # dbias onto dphi
    assert f(p, ws=A[4]) == 6                          # workspace onto dH
    assert lib.mhc_pre_bwd_workspace_size(None) == 0
    assert lib.mhc_pre_bwd_workspace_size(ctypes.byref(_params(n=3))) == 0


def test_pre_bwd_ex_argument_checks(lib):
    """mhc_pre_bwd_ex: G must not overlap an output and must be aligned;
    mhc_post_bwd accepts a NULL dX (the whole-dX pair)."""
    p = _params()
    need = lib.mhc_pre_bwd_workspace_size(ctypes.byref(p))
    far = [0x1000000000 * (k + 1) for k in range(12)]

    def f(G, dX=far[7]):
        return lib.mhc_pre_bwd_ex(ctypes.byref(p), far[0], far[1], far[2], far[3], far[4], G, dX, far[8], far[9],
                                  far[10], far[11], need, None)
    assert f(far[5] + 8) == 4                          # G misaligned
    assert f(far[7]) == 6                              # G onto dX
    assert f(far[8]) == 6                              # G onto dphi
    assert lib.mhc_post_bwd_ex(ctypes.byref(p), far[0], far[1], far[2], far[3], None, None, far[6], None, 0,
                               None) == 1              # dY NULL is still refused
    assert lib.mhc_post_bwd_ex(ctypes.byref(p), far[0], far[1], far[2], far[3], None, far[3], far[6], None, 0,
                               None) == 6              # dY onto G, with dX NULL


def test_post_pre_argument_checks(lib):
    p = _params()
    need = lib.mhc_pre_workspace_size(ctypes.byref(p))

    def f(p, X=A[0], Y=A[1], H=A[2], O=A[3], phi=A[4], bias=A[5], h=A[6], Hn=A[7], ws=A[7] + (1 << 24), nb=None):
        nb = need if nb is None else nb
        return lib.mhc_post_pre(ctypes.byref(p), X, Y, H, O, phi, bias, h, Hn, ws, nb, None)
    assert f(_params(n=3)) == 5
    assert f(p, phi=None) == 1
    assert f(p, ws=None) == 7
    assert f(p, nb=need - 1) == 7
    assert f(p, O=A[0] + 512) == 6                     # partial overlap with X
    assert f(p, h=A[1]) == 6                           # h onto Y
    assert f(p, Hn=A[6]) == 6                          # H_next onto h
    assert f(p, ws=A[2]) == 6                          # workspace onto the previous maps
    assert f(p, X=A[0] + 4) == 4
    assert f(_params(T=0), X=None) == 0

    def fx(algo, O=A[3]):
        used = ctypes.c_int32(-7)
        st = lib.mhc_post_pre_ex(ctypes.byref(p), A[0], A[1], A[2], O, A[4], A[5], A[6], A[7], A[7] + (1 << 24),
                                 need, algo, ctypes.byref(used), None)
        return st, used.value
    assert fx(7) == (2, 1)                             # unknown algorithm; *algo_used reset to the two-pass code
    assert fx(2, O=A[0]) == (6, 1)                     # the single pass needs X_{l+1} apart from X
    assert fx(3, O=A[0]) == (6, 1)


def test_maps_field(lib):
    import mhc_hyper_connections_amd as m
    assert _pre(lib, _params(maps=7)) == 2                          # unknown form of the maps
    p = _params(maps=m.MAPS_HC)
    assert lib.mhc_pre_bwd(ctypes.byref(p), *A[:8], A[7] + 4096, A[7] + 8192,
                           lib.mhc_pre_bwd_workspace_size(ctypes.byref(p)), None) == 5   # no HC backward
    assert ctypes.sizeof(m.Params) == 48


def test_pre_noalloc_host_checks(lib):
    """mhc_pre_noalloc refuses, before anything reaches a device, what mhc_pre
    refuses, and a call whose scratch would exceed its static buffer."""
    import mhc_hyper_connections_amd as m
    call = lambda p, ptrs=A[:5]: lib.mhc_pre_noalloc(None if p is None else ctypes.byref(p), *ptrs, None)
    assert call(None) == 1                                                  # NULL params
    assert call(_params(n=3)) == 5                                          # unsupported n
    assert call(_params(T=-1)) == 2
    assert call(_params(), (A[0], None, A[2], A[3], A[4])) == 1             # NULL phi
    assert call(_params(T=0), (None,) * 5) == 0                             # T = 0 is a no-op
    big = _params(T=40000, n=4, d=4096)
    far = [0x1000000000 * (k + 1) for k in range(5)]                       # 64 GiB apart: no overlap
    assert lib.mhc_pre_workspace_size(ctypes.byref(big)) > m.PRE_NOALLOC_SCRATCH_BYTES
    assert call(big, far) == 9                                              # MHC_ERR_SCRATCH
    fits = _params(T=16384, n=4, d=4096)
    assert lib.mhc_pre_workspace_size(ctypes.byref(fits)) <= m.PRE_NOALLOC_SCRATCH_BYTES
