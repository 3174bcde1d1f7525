"""GPU check of flarepp_mix_noalloc, the mixer entry point that allocates nothing (its workspace is
the library's static device scratch), through the C ABI: two calls in a row, the second on a
smaller problem, each bit for bit equal to flarepp_mix_ws on the same inputs (the same kernels and
launch plan, so the same arithmetic), and the first also against the float64 oracle on sampled
slices at the bf16 bar."""
import numpy as np
import pytest

from gpu_util import oracle_head, say, slice_err, tol, to_device
from workloads import make_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_routing_amd as fl
    fl.lib()  # fails loudly when the library is missing


def _args(dev):
    return dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"]


def test_noalloc_matches_the_workspace_entry_point_twice():
    import rank_latent_routing_amd as fl
    # The larger problem first (the M = 256 workload shape, 18 MiB of workspace), then a smaller one
    # (the M = 64 mesh workload, reduced), which runs on what the first call left in the scratch.
    cases = [make_workload(4, B=2, H=8, N=65536), make_workload(2, B=2, H=4, N=5000)]
    for i, w in enumerate(cases):
        dt = fl.FLAREPP_BF16 if w.dtype == "bf16" else fl.FLAREPP_FP32
        need = fl.flarepp_workspace_bytes(w.B, w.H, w.N, w.M, w.D, dt)
        say(f"[noalloc] call {i}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}, workspace {need} bytes")
        assert 0 < need <= fl.FLAREPP_NOALLOC_SCRATCH_BYTES
        dev = to_device(w)
        out = torch.empty_like(dev["K"])
        fl.flarepp_mix_noalloc(*_args(dev), out=out)
        ref = fl.flarepp_mix_ws(*_args(dev))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"call {i} differs from flarepp_mix_ws"
        if i == 0:
            Y = out.float().cpu().numpy().astype(np.float64)
            for b, h in ((0, 0), (1, 7)):
                e = slice_err(Y[b, h], oracle_head(w, b, h)["Y"], w.dtype)
                say(f"[noalloc] slice ({b}, {h}): {e:.4g} of RMS")
                assert e <= tol(w.dtype)
