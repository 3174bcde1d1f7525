"""GPU parity of simplified FLARE++ (Appendix A.8, Eq. 20; flarepp_mix_simplified through the C ABI)
against the float64 oracle's simplified_mix_head, with the forward pass's bars: fp32
max|Y - Y_ref| / max|Y_ref| <= 1e-5, bf16 max|Y - Y_ref| <= 2e-2 RMS(Y_ref), per (b, h) slice."""
import numpy as np
import pytest

import oracle
from gpu_util import say, slice_err, tol
from workloads import make_synthesis_values, make_workload, to_float64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_routing_amd as fl
    fl.lib()  # fails loudly when the library is missing


def _dev(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _run(w, Sv, workspace=False):
    import rank_latent_routing_amd as fl
    ws = None
    if workspace:
        ws = torch.empty(max(fl.flarepp_workspace_bytes(w.B, w.H, w.N, w.M, w.D, 1 if w.dtype == "bf16" else 0), 1),
                         dtype=torch.uint8, device="cuda")
    out = fl.flarepp_mix_simplified(_dev(w.K, w.dtype), _dev(w.V, w.dtype), _dev(w.S, w.dtype), _dev(Sv, w.dtype),
                                    _dev(w.Qseed, w.dtype), workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _check(w, heads=None, block=None, label=""):
    say(f"[simplified] {label or w.name}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}")
    Sv = make_synthesis_values(w)
    Y = _run(w, Sv)
    assert np.isfinite(Y).all()
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    worst = 0.0
    for b, h in pairs:
        ref = oracle.simplified_mix_head(to_float64(w.K[b, h], w.dtype), to_float64(w.V[b, h], w.dtype), to_float64(w.S[b, h], w.dtype),
                                         to_float64(Sv[b, h], w.dtype), to_float64(w.Qseed[h], w.dtype), block)["Y"]
        worst = max(worst, slice_err(Y[b, h], ref, w.dtype))
    say(f"[simplified] {label or w.name}: worst {worst:.3g} (bar {tol(w.dtype)})")
    assert worst <= tol(w.dtype)
    return Y, Sv


def test_simplified_cfg1_fp32():
    _check(make_workload(1))


@pytest.mark.parametrize("N,M,D", [(1, 1, 16), (3001, 33, 32), (777, 300, 32)])
def test_simplified_fp32_shapes(N, M, D):
    _check(make_workload(1, N=N, M=M, D=D, seed=500 + N + M), label=f"fp32 N={N} M={M} D={D}")


def test_simplified_cfg2_bf16():
    _check(make_workload(2, B=2, H=2, N=5000))


@pytest.mark.parametrize("M", [100, 256, 512])
def test_simplified_bf16_latent_counts(M):
    _check(make_workload(4, B=1, H=2, N=20000, M=M, seed=600 + M), label=f"bf16 M={M}")


def test_simplified_cfg5_full_size_one_head():
    # The 1M-token workload at its full size; the oracle takes head 0 in token blocks.
    w = make_workload(5)
    _check(w, heads=[(0, 0)], block=65536, label="cfg5 full, head 0")


def test_simplified_entry_points_agree_and_deterministic():
    w = make_workload(4, B=1, H=2, N=5000, M=200, seed=21)
    Sv = make_synthesis_values(w)
    a, b, c = _run(w, Sv), _run(w, Sv, workspace=True), _run(w, Sv)
    assert np.array_equal(a, b) and np.array_equal(a, c)
