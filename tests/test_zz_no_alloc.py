"""mhc_pre_noalloc: mhc_pre on the library's static per-GPU scratch (no
workspace, no allocation) against mhc_pre with its own workspace.

Two calls in a row through the C ABI, the second on a smaller input, each
compared with mhc_pre on the same inputs: both take MHC_PRE_AUTO's form (the
single pass at T = 16384, d = 4096; the small-T two-pass form at T = 300,
d = 2048), so the results must be the same bits.  A call that needs more
scratch than the static array holds is refused before anything runs.
"""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connections_amd as m
    m.load_library()
    return m


def _inputs(T, n, d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    m = n * n + 2 * n
    X = torch.randn(T, n, d, device="cuda", generator=g).to(torch.bfloat16)
    phi = torch.randn(n * d, m, device="cuda", generator=g) * 0.02
    bias = torch.randn(m, device="cuda", generator=g) * 0.1
    return X, phi, bias


def test_noalloc_matches_mhc_pre(mhc):
    alpha = (0.01, 0.01, 0.01)
    for k, (T, n, d, form) in enumerate(((16384, 4, 4096, mhc.PRE_ONE_PASS), (300, 4, 2048, mhc.PRE_TWO_PASS))):
        print(f"[noalloc] call {k}: T={T} n={n} d={d}", flush=True)
        X, phi, bias = _inputs(T, n, d, 500 + k)
        h, H = mhc.pre_noalloc(X, phi, bias, alpha=alpha)
        torch.cuda.synchronize()
        h_ref, H_ref, used = mhc.pre_ex(X, phi, bias, mhc.PRE_AUTO, alpha=alpha)
        torch.cuda.synchronize()
        assert used == form
        assert torch.equal(h, h_ref), f"call {k}: h differs from mhc_pre"
        assert torch.equal(H, H_ref), f"call {k}: H differs from mhc_pre"


def test_noalloc_refuses_calls_beyond_its_scratch(mhc):
    T, n, d = 40000, 4, 4096
    assert mhc.pre_workspace_size(T, n, d, mhc.MHC_BF16) > mhc.PRE_NOALLOC_SCRATCH_BYTES
    X = torch.empty((T, n, d), dtype=torch.bfloat16, device="cuda")
    phi = torch.zeros((n * d, n * n + 2 * n), device="cuda")
    bias = torch.zeros(n * n + 2 * n, device="cuda")
    with pytest.raises(mhc.MhcError) as ei:
        mhc.pre_noalloc(X, phi, bias)
    assert ei.value.status == 9
