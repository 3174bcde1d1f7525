"""Streams and HIP graphs. The workspace entry points inside HIP graphs: flarepp_mix_ws, flarepp_mix_backward_ws and
flarepp_block_ws enqueue kernels only (no allocation, no memset, no host synchronization), so a
caller can capture them once and replay them. Each graph is replayed several times with eager calls
of the library and synchronizations in between, and every replay must equal the eager result bit
for bit (the kernels are deterministic). Calls on a stream the caller created match the default
stream's results."""
import numpy as np
import pytest

from gpu_util import say, to_device
from workloads import make_block_inputs, make_cotangent, make_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_routing_amd as fl
    fl.lib()  # fails loudly when the library is missing


def _t(arr, dtype):
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _capture(fn):
    """Warm `fn` up on a side stream (default priority), then capture it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, outs, refs, eager_between):
    for i in range(4):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i}"
        eager_between()
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_mixer_graph_replays(dtype):
    import rank_latent_routing_amd as fl
    w = make_workload(2, B=1, H=2, N=5000, dtype=dtype)
    say(f"[graph] mixer {w.name} {dtype} N={w.N}")
    dev = to_device(w)
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    ws = torch.empty(fl.flarepp_workspace_bytes(w.B, w.H, w.N, w.M, w.D, 1 if dtype == "bf16" else 0),
                     dtype=torch.uint8, device="cuda")
    ref = fl.flarepp_mix_ws(*args, workspace=ws).clone()
    out = torch.empty_like(ref)
    g = _capture(lambda: fl.flarepp_mix_ws(*args, out=out, workspace=ws))
    # Between replays: another problem through the same workspace.
    w2 = make_workload(4, B=1, H=2, N=3000, M=40, seed=5, dtype=dtype)
    d2 = to_device(w2)
    ws2_need = fl.flarepp_workspace_bytes(w2.B, w2.H, w2.N, w2.M, w2.D, 1 if dtype == "bf16" else 0)
    ws2 = ws if ws2_need <= ws.numel() else torch.empty(ws2_need, dtype=torch.uint8, device="cuda")
    other = lambda: fl.flarepp_mix_ws(d2["K"], d2["V"], d2["S"], d2["Qseed"], d2["Qf"], d2["g"], workspace=ws2)
    _replays_match(g, [out], [ref], other)


def test_backward_graph_replays():
    import rank_latent_routing_amd as fl
    w = make_workload(4, B=1, H=2, N=3000, M=100, seed=7)
    say(f"[graph] backward {w.name} N={w.N}")
    dev = to_device(w)
    dY = _t(make_cotangent(w), w.dtype)
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"], dY)
    ws = torch.empty(fl.flarepp_backward_workspace_bytes(w.B, w.H, w.N, w.M, w.D, 1), dtype=torch.uint8,
                     device="cuda")
    ref = {k: v.clone() for k, v in fl.flarepp_mix_backward(*args, workspace=ws).items()}
    grads = {k: torch.empty_like(v) for k, v in ref.items()}
    g = _capture(lambda: fl.flarepp_mix_backward(*args, grads=grads, workspace=ws))
    other = lambda: fl.flarepp_mix_ws(*args[:6])
    keys = sorted(ref)
    _replays_match(g, [grads[k] for k in keys], [ref[k] for k in keys], other)


def test_block_graph_replays():
    import rank_latent_routing_amd as fl
    w = make_workload(2, B=1, H=8, N=3000, M=48, seed=3)
    say(f"[graph] block {w.name} N={w.N}")
    bi = make_block_inputs(w, seed=4)
    X = _t(bi.X, w.dtype)
    W = [_t(m.T, w.dtype) for m in (bi.Wk, bi.Wv, bi.Ws, bi.Wo)]
    vec = {k: _t(getattr(bi, k), w.dtype) for k in ("bk", "bv", "bs", "bo", "nq", "nk")}
    Qs, Qf = _t(w.Qseed, w.dtype), _t(w.Qf, w.dtype)
    gamma = torch.from_numpy(bi.gamma).cuda()
    ws = torch.empty(fl.flarepp_block_workspace_bytes(w.B, w.H, w.N, w.M, w.D, 1), dtype=torch.uint8, device="cuda")
    call = lambda out: fl.flarepp_block(X, *W, Qs, Qf, gamma, out=out, workspace=ws, **vec)
    ref = call(None).clone()
    out = torch.empty_like(ref)
    g = _capture(lambda: call(out))
    other = lambda: fl.flarepp_out_project(torch.ones((w.B, w.H, w.N, w.D), dtype=torch.bfloat16, device="cuda"), W[3])
    _replays_match(g, [out], [ref], other)


def test_calls_on_a_caller_stream_match_the_default_stream():
    # The stream argument: the mixer and its backward enqueued on a stream the caller created (with
    # other work queued ahead of them there) give the default stream's results bit for bit.
    import rank_latent_routing_amd as fl
    w = make_workload(4, B=1, H=2, N=4000, M=96, seed=13)
    say(f"[stream] {w.name} N={w.N}")
    dev = to_device(w)
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    dY = _t(make_cotangent(w), w.dtype)
    ref = fl.flarepp_mix_ws(*args).clone()
    gref = {k: v.clone() for k, v in fl.flarepp_mix_backward(*args, dY).items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    busy = torch.empty(2 ** 24, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        busy.fill_(1.0)  # queued ahead of the library's kernels on the same stream
        out = torch.empty_like(ref)
        fl.flarepp_mix_ws(*args, out=out, stream=s)
        grads = fl.flarepp_mix_backward(*args, dY, stream=s)
    s.synchronize()
    assert torch.equal(out, ref)
    for k in gref:
        assert torch.equal(grads[k], gref[k]), k
