"""GPU parity of the HIP mixer backward pass (flarepp_mix_backward, through the C ABI) against the
float64 oracle's mix_head_backward: the SDPA backward of Appendix B.5 (Eq. 46-49) applied to the
decode, encode and synthesis calls (Section 3.2, Eq. 6 and Eq. 8), through the gate (Eq. 7) and
N0 (Eq. 5).

Bars, per tensor: fp32 max|x - x_ref| / max|x_ref| <= 1e-5 (the forward pass's bar). bf16: every
element within 2e-2 RMS(x_ref) + 2^-8 |x_ref|. The cotangents are stored in bf16, whose rounding to
nearest alone moves an element by up to 2^-8 of itself (the unit roundoff of an 8-bit significand),
and they are heavy-tailed (single elements reach 30 times the tensor's RMS), so a bar on 2e-2 RMS
alone would fail on storage; 2^-8 |x_ref| is that storage rounding (the forward's bar for its
heavy-tailed outputs has the same form).
dK, dV, dS per (b, h) slice; dQseed and dQf (summed over the batch) per head; dg per head against
sum_b sum_{m,d} |dQ Qd|, the size of the terms it sums, so that cancellation among them neither
loosens nor tightens the bar.
"""
import numpy as np
import pytest

import oracle
from gpu_util import say, slice_err, tol, to_device
from workloads import make_cotangent, make_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_routing_amd as fl
    fl.lib()  # fails loudly when the library is missing


def _device(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def run_backward(w, dY, workspace=False, grads=None):
    import rank_latent_routing_amd as fl
    dev = to_device(w)
    dy = _device(dY, w.dtype)
    ws = None
    if workspace:
        need = fl.flarepp_backward_workspace_bytes(w.B, w.H, w.N, w.M, w.D, 1 if w.dtype == "bf16" else 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = fl.flarepp_mix_backward(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"], dy,
                                  grads=grads, workspace=ws)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}


def oracle_backward(w, dY):
    """The oracle's cotangents, slice by slice, plus the dg scale sum_b sum |dQ Qd| per head."""
    K, V, S = w.f64("K"), w.f64("V"), w.f64("S")
    Qs, Qf = w.f64("Qseed"), w.f64("Qf")
    from workloads import to_float64
    dy = to_float64(dY, w.dtype)
    out = {"dK": np.zeros(K.shape), "dV": np.zeros(K.shape), "dS": np.zeros(K.shape),
           "dQseed": np.zeros(Qs.shape), "dQf": np.zeros(Qs.shape), "dg": np.zeros(w.H),
           "dg_scale": np.zeros(w.H)}
    for b in range(w.B):
        for h in range(w.H):
            g = float(w.g[h])
            r = oracle.mix_head_backward(K[b, h], V[b, h], S[b, h], Qs[h], Qf[h], g, dy[b, h])
            Qd = oracle.synthesis(Qs[h], S[b, h])
            out["dK"][b, h], out["dV"][b, h], out["dS"][b, h] = r["dK"], r["dV"], r["dS"]
            out["dQseed"][h] += r["dQseed"]
            out["dQf"][h] += r["dQf"]
            out["dg"][h] += r["dg"]
            out["dg_scale"][h] += np.abs(r["dQ"] * Qd).sum()
    return out


def _err(got, ref, dtype):
    if dtype == "fp32":
        return slice_err(got, ref, dtype)
    excess = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)
    return max(float(excess.max()), 0.0) / max(np.sqrt(np.mean(ref * ref)), 1e-30)


def run_saved(w, dY):
    """flarepp_mix_forward_saved, then flarepp_mix_backward_saved from its workspace."""
    import rank_latent_routing_amd as fl
    dev = to_device(w)
    dy = _device(dY, w.dtype)
    need = fl.flarepp_backward_workspace_bytes(w.B, w.H, w.N, w.M, w.D, 1 if w.dtype == "bf16" else 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    fl.flarepp_mix_forward_saved(*args, workspace=ws)
    out = fl.flarepp_mix_backward_saved(*args, dy, workspace=ws)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}


def _check(w, dY=None, label="", bar=None, runner=None):
    say(f"[bwd] {label or w.name}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}")
    dY = make_cotangent(w) if dY is None else dY
    got = (runner or run_backward)(w, dY)
    for k, v in got.items():
        assert np.isfinite(v).all(), k
    ref = oracle_backward(w, dY)
    worst = {}
    for k in ("dK", "dV", "dS"):
        for b in range(w.B):
            for h in range(w.H):
                worst[k] = max(worst.get(k, 0.0), _err(got[k][b, h], ref[k][b, h], w.dtype))
    for k in ("dQseed", "dQf"):
        for h in range(w.H):
            worst[k] = max(worst.get(k, 0.0), _err(got[k][h], ref[k][h], w.dtype))
    worst["dg"] = float(np.max(np.abs(got["dg"] - ref["dg"]) / np.maximum(ref["dg_scale"], 1e-30)))
    bar = tol(w.dtype) if bar is None else bar
    say(f"[bwd] {label or w.name}: worst {worst} (bar {bar})")
    for k, e in worst.items():
        assert e <= bar, (k, e)
    return got, ref


def test_bwd_cfg1_fp32():
    _check(make_workload(1))


@pytest.mark.parametrize("N,M,D", [(64, 1, 16), (100, 33, 32), (3001, 17, 16), (777, 100, 32), (2048, 512, 32)])
def test_bwd_fp32_shapes(N, M, D):
    _check(make_workload(1, N=N, M=M, D=D, seed=300 + N + M), label=f"fp32 N={N} M={M} D={D}")


@pytest.mark.parametrize("M,D", [(1, 16), (40, 32)])
def test_bwd_single_token_closed_form(M, D):
    # With one token every token-axis softmax is 1: Z_m = V and Qd_m = N0(S) for every latent, so
    # Y = V whatever K, S, Qseed, Qf and g hold. Hence dV = dY and every other cotangent is zero.
    w = make_workload(1, B=2, N=1, M=M, D=D, seed=11 + M)
    dY = make_cotangent(w)
    say(f"[bwd] single token M={M} D={D}")
    got = run_backward(w, dY)
    dy = w.f64("K") * 0 + dY.astype(np.float64)
    assert np.abs(got["dV"] - dy).max() <= 1e-6 * np.abs(dy).max()
    for k in ("dK", "dS", "dQseed", "dQf", "dg"):
        assert np.abs(got[k]).max() <= 1e-5 * np.abs(dy).max(), k


def test_bwd_cfg2_bf16():
    _check(make_workload(2, B=2, H=2, N=5000))


def test_bwd_cfg3_bf16_gate_zero_head():
    w = make_workload(3, B=2, H=2, N=2000)
    got, _ = _check(w)
    # Head 0 has g = 0: the synthesis call does not reach the output, so its cotangents vanish
    # exactly (Eq. 7: Q = N0(Qf) + g Qd).
    assert not got["dS"][:, 0].any()
    assert not got["dQseed"][0].any()
    assert got["dS"][:, 1].any() and got["dQseed"][1].any()


@pytest.mark.parametrize("M", [100, 300, 512])
def test_bwd_bf16_latent_counts(M):
    _check(make_workload(4, B=1, H=2, N=20000, M=M, seed=400 + M), label=f"bf16 M={M}")


def test_bwd_bf16_gaussian_d16_ragged():
    _check(make_workload(1, B=2, H=2, N=3001, M=77, D=16, dtype="bf16", seed=77), label="bf16 gauss D=16")


def test_bwd_peaked():
    _check(make_workload(4, peaked=True, B=1, H=2, N=20000), label="cfg4 peaked")


def test_bwd_cfg5_shape_one_head():
    # cfg5's head shape (M = 512, D = 32, surface inputs) at 65536 tokens.
    _check(make_workload(5, H=1, N=65536), label="cfg5 N=65536 H=1")


@pytest.mark.parametrize("tok,lat", [("32", "8"), ("2048", "4096")])
def test_bwd_launch_plans(monkeypatch, tok, lat):
    # Workgroup counts other than the defaults: one token chunk per latent group (every reduction
    # sums one partial per entry, one wave per 64 entries) or 79 chunks (the four waves of a
    # reduction block split them), with few or many token-side workgroups.
    monkeypatch.setenv("FLAREPP_BWD_TOKEN_WORKGROUPS", tok)
    monkeypatch.setenv("FLAREPP_BWD_LATENT_WORKGROUPS", lat)
    w = make_workload(4, B=2, H=2, N=20000, M=300, seed=78)
    _check(w, label=f"bwd plan tok={tok} lat={lat}")
    _check(w, label=f"bwd plan tok={tok} lat={lat} saved", runner=run_saved)


def test_bwd_full_cfg5_one_head():
    # The 1M-token workload at its full size (B = 1, H = 8, N = 2^20, M = 512), in the launch
    # configuration the benchmark times; head 3 against the token-blocked oracle: dK, dV and dS at
    # every token, dQseed, dQf and dg.
    import rank_latent_routing_amd as fl
    from workloads import to_float64
    w = make_workload(5)
    dY = make_cotangent(w)
    h = 3
    say(f"[bwd] cfg5 full: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}, GPU")
    dev = to_device(w)
    out = fl.flarepp_mix_backward(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"],
                                  _device(dY, w.dtype))
    torch.cuda.synchronize()
    for k, v in out.items():
        assert bool(torch.isfinite(v.float()).all()), k
    got = {k: out[k][0, h].float().cpu().numpy().astype(np.float64) for k in ("dK", "dV", "dS")}
    got.update({k: out[k][h].float().cpu().numpy().astype(np.float64) for k in ("dQseed", "dQf")})
    got["dg"] = float(out["dg"][h])
    del out, dev
    say(f"[bwd] cfg5 full: oracle, head {h}")
    f = lambda a: to_float64(a, w.dtype)
    ref = oracle.mix_head_backward_blocked(f(w.K[0, h]), f(w.V[0, h]), f(w.S[0, h]), f(w.Qseed[h]), f(w.Qf[h]),
                                           float(w.g[h]), f(dY[0, h]), 65536)
    worst = {k: _err(got[k], ref[k], w.dtype) for k in ("dK", "dV", "dS", "dQseed", "dQf")}
    worst["dg"] = abs(got["dg"] - ref["dg"]) / np.abs(ref["dQ"] * ref["Qd"]).sum()
    say(f"[bwd] cfg5 full, head {h}: worst {worst} (bar {tol(w.dtype)})")
    for k, e in worst.items():
        assert e <= tol(w.dtype), (k, e)


def test_bwd_saved_full_cfg5_bitwise():
    # The benchmark times flarepp_mix_forward_saved + flarepp_mix_backward_saved at the 1M-token
    # workload; at that size they return the self-contained backward's cotangents bit for bit
    # (which test_bwd_full_cfg5_one_head checks against the oracle), and the saved forward's output
    # is within the forward's bar of the inference forward's.
    import rank_latent_routing_amd as fl
    w = make_workload(5)
    dY = make_cotangent(w)
    say(f"[bwd] cfg5 full, saved state against recompute: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}")
    dev = to_device(w)
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    dy = _device(dY, w.dtype)
    ref = fl.flarepp_mix_backward(*args, dy)
    need = fl.flarepp_backward_workspace_bytes(w.B, w.H, w.N, w.M, w.D, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_saved = fl.flarepp_mix_forward_saved(*args, workspace=ws)
    got = fl.flarepp_mix_backward_saved(*args, dy, workspace=ws)
    y = fl.flarepp_mix(*args)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    d = (y_saved.float() - y.float()).abs().max().item()
    rms = y.float().pow(2).mean().sqrt().item()
    say(f"[bwd] cfg5 full: saved == recompute bitwise; saved forward against forward {d / rms:.4g} of RMS")
    assert d <= 2 * tol(w.dtype) * rms


def test_bwd_determinism_and_entry_points_agree():
    w = make_workload(4, B=1, H=2, N=5000, M=200, seed=9)
    dY = make_cotangent(w)
    a = run_backward(w, dY)
    b = run_backward(w, dY, workspace=True)
    c = run_backward(w, dY)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k


def test_bwd_empty_problem_zeroes_parameter_cotangents():
    import rank_latent_routing_amd as fl
    w = make_workload(1, N=0)
    dev = to_device(w)
    dy = torch.empty_like(dev["K"])
    grads = {"dK": torch.empty_like(dev["K"]), "dV": torch.empty_like(dev["K"]), "dS": torch.empty_like(dev["K"]),
             "dQseed": torch.full_like(dev["Qseed"], 7.0), "dQf": torch.full_like(dev["Qf"], 7.0),
             "dg": torch.full_like(dev["g"], 7.0)}
    fl.flarepp_mix_backward(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"], dy, grads=grads)
    torch.cuda.synchronize()
    for k in ("dQseed", "dQf", "dg"):
        assert not grads[k].any(), k


@pytest.fixture
def force_exact():
    import rank_latent_routing_amd as fl
    prev = fl.flarepp_debug_force_exact(True)
    yield
    fl.flarepp_debug_force_exact(prev)


@pytest.mark.parametrize("cfg,kw", [(1, {}), (4, dict(B=1, H=2, N=5000, M=200, seed=21))])
def test_bwd_running_maximum_passes(force_exact, cfg, kw):
    # With the test hook the recomputed forward and the decode statistics take their running-maximum
    # passes, the fallbacks of their zero-shift passes.
    _check(make_workload(cfg, **kw), label=f"bwd running maxima cfg{cfg}")


def _routing_logits(w, b, h):
    """The decode logits log2(e) K Q^T / sqrt(D) of slice (b, h) and the sums log2(e) |K| |Q|^T /
    sqrt(D) of their terms' magnitudes."""
    K, S = w.f64("K")[b, h], w.f64("S")[b, h]
    Q = oracle.gate(w.f64("Qf")[h], oracle.synthesis(w.f64("Qseed")[h], S), float(w.g[h]))
    c = np.log2(np.e) / np.sqrt(K.shape[1])
    return (K @ Q.T) * c, (np.abs(K) @ np.abs(Q).T) * c


def _decode_rows_out_of_range(w, b=0, h=0):
    """Fraction of tokens whose zero-shift decode row sum, sum_m 2^(log2(e) q_m.k/sqrt(D)), falls
    outside [2^-80, 2^100]: the tokens whose waves take the running-maximum statistics."""
    L, _ = _routing_logits(w, b, h)
    m = L.max(axis=1)
    lsum = m + np.log2(np.exp2(L - m[:, None]).sum(axis=1))
    return float(((lsum > 100.0) | (lsum < -80.0)).mean())


@pytest.mark.parametrize("dtype,big", [("fp32", 36.0), ("bf16", 40.0)])
def test_bwd_zero_shift_and_running_maximum_mixed(dtype, big):
    # Large keys in two token ranges: the token waves that hold them take the running-maximum
    # decode statistics (and the recompute's chunks that hold them the running-maximum pass), all
    # others keep the zero-shift result.
    w = make_workload(4, B=1, H=2, N=20000, dtype=dtype)
    from workloads.gen import _store
    K = w.f64("K")
    K[:, :, 17000:17500] *= big
    K[:, :, 8000:8100] *= big
    w.K = _store(K, dtype)
    assert 0.0 < _decode_rows_out_of_range(w, 0, 0) < 0.03
    bar = None
    if dtype == "fp32":
        # fp32 logits carry a rounding error of about sqrt(D) 2^-24 sum_d |q_d k_d| (log2 units; the
        # dot product's accumulation), which moves a probability by ln 2 times that. The large keys
        # put that sum near 255, beyond what the plain 1e-5 bar allows: add it.
        big_sum = max(float(_routing_logits(w, 0, h)[1].max()) for h in range(w.H))
        bar = 1e-5 + np.log(2.0) * 2.0 ** -24 * np.sqrt(w.D) * big_sum
    _check(w, label=f"bwd mixed {dtype}", bar=bar)


@pytest.mark.parametrize("name,rows,scale", [("V", (5000, 5100), 2.0 ** 17), ("V", None, 2.0 ** -10),
                                             ("K", (8000, 8100), 2.0 ** 15)])
def test_bwd_bf16_token_values_beyond_fp16(name, rows, scale):
    # The bf16 encode call's token-side products take K and V in fp16, exact for magnitudes in
    # [2^-14, 2^15). A 32-token group whose values leave that range takes them scaled by a power of
    # two and takes the scale back out of its products: values of 2^17 in one token range (those
    # groups only), values below 2^-6 everywhere (every group), keys of 2^15 in one token range.
    # The oracle sees the same bf16 values.
    w = make_workload(4, B=1, H=2, N=20000, seed=31)
    from workloads.gen import _store
    X = w.f64(name)
    if rows is None:
        X *= scale
    else:
        X[:, :, rows[0]:rows[1]] *= scale
    setattr(w, name, _store(X, w.dtype))
    label = f"bwd bf16 {name} x{scale:g}" + (f" on tokens {rows[0]}-{rows[1]}" if rows else "")
    if name == "V":
        _check(w, label=label)
        return
    # Keys of 2^15 put routing logits near 4e4 (log2 units). The bf16 pair that carries c*Q to every
    # kernel (about 16 significant bits) then moves logits by up to about 0.3, so the cotangents
    # that go through those softmaxes' probabilities leave the bar in every kernel alike. Checked
    # here: every output finite, and dK (the product the scaled keys feed) at the bar.
    say(f"[bwd] {label}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}")
    dY = make_cotangent(w)
    got = run_backward(w, dY)
    for k, v in got.items():
        assert np.isfinite(v).all(), k
    ref = oracle_backward(w, dY)
    worst = max(_err(got["dK"][0, h], ref["dK"][0, h], w.dtype) for h in range(w.H))
    say(f"[bwd] {label}: worst dK {worst} (bar {tol(w.dtype)})")
    assert worst <= tol(w.dtype)


def test_bwd_bf16_seeds_beyond_fp16():
    # The bf16 synthesis call's token-side products take the seeds in fp16, exact below 2^15; a head
    # whose seeds reach 2^15 takes them scaled by a power of two, with the score product's start
    # values scaled alike. One seed row of head 0 at 2^15 sends that head there; its synthesis
    # logits for that row reach about 4e4 (log2 units), where the pairs carrying c N0(S) move them
    # by up to about 0.3, as with keys of 2^15 (above). Checked: every output finite, and head 1
    # (ordinary seeds) at the bars.
    w = make_workload(3, B=1, H=2, N=3000, M=64, seed=17)
    from workloads.gen import _store
    Qs = w.f64("Qseed")
    Qs[0, 5] *= 2.0 ** 15
    w.Qseed = _store(Qs, w.dtype)
    say(f"[bwd] bf16 seeds at 2^15 in head 0: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}")
    dY = make_cotangent(w)
    got = run_backward(w, dY)
    for k, v in got.items():
        assert np.isfinite(v).all(), k
    ref = oracle_backward(w, dY)
    worst = {k: _err(got[k][0, 1], ref[k][0, 1], w.dtype) for k in ("dK", "dV", "dS")}
    worst.update({k: _err(got[k][1], ref[k][1], w.dtype) for k in ("dQseed", "dQf")})
    say(f"[bwd] bf16 seeds at 2^15, head 1: worst {worst} (bar {tol(w.dtype)})")
    for k, e in worst.items():
        assert e <= tol(w.dtype), (k, e)


@pytest.mark.parametrize("scale", [2.0 ** -24, 2.0 ** 16])
def test_bwd_bf16_cotangent_scales(scale):
    # Cotangents far from unit size (a loss's gradients are often tiny): the bf16 kernels that take
    # fp16 operands scale dY, dZ, G and dS into fp16's range by powers of two from their maxima, so
    # the cotangents, which are linear in dY, meet the same relative bars at any scale.
    w = make_workload(4, B=1, H=2, N=20000, seed=23)
    from workloads.gen import _store
    from workloads import to_float64
    dY = _store(to_float64(make_cotangent(w), w.dtype) * scale, w.dtype)
    _check(w, dY=dY, label=f"bwd bf16 dY x{scale:g}")


@pytest.mark.parametrize("dtype,seeds", [("bf16", 3.0), ("bf16", 6.0), ("fp32", 6.0)])
def test_bwd_seed_scales(dtype, seeds):
    # The seeds' learned scale sets the synthesis call's temperature (Appendix A.3, Eq. 14). At x6
    # every synthesis row is nearly one-hot over the tokens, so its cotangent P (dP - c) is a
    # difference of nearly equal terms, and the routing queries inherit the synthesis output's
    # rounding at full weight.
    w = make_workload(3, B=1, H=2, N=3000, M=64, dtype=dtype, seed=13)
    from workloads.gen import _store
    w.Qseed = _store(w.f64("Qseed") * seeds, dtype)
    _check(w, label=f"bwd seeds x{seeds:g} {dtype}")


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("scale", [8.0, 24.0])
def test_bwd_saturated_softmaxes(dtype, scale, saved):
    # Keys scaled on every token (Appendix B.5, Eq. 46-49 in the saturated regime): at x24 the
    # routing logits reach about 200 (log2 units), every softmax row is nearly one-hot, and each
    # score cotangent P (dP - c) is a difference of nearly equal terms. The bf16 bars hold as they
    # stand; fp32 adds the logits' accumulation error, as in the mixed case above.
    w = make_workload(3, B=1, H=2, N=3000, M=64, dtype=dtype, seed=11)
    from workloads.gen import _store
    w.K = _store(w.f64("K") * scale, dtype)
    bar = None
    if dtype == "fp32":
        big_sum = max(float(_routing_logits(w, 0, h)[1].max()) for h in range(w.H))
        bar = 1e-5 + np.log(2.0) * 2.0 ** -24 * np.sqrt(w.D) * big_sum
    # The saved path reads the softmax statistics the forward kept: the saturated rows are where
    # those must still reproduce the recomputed ones.
    _check(w, label=f"bwd saturated x{scale:g} {dtype}{' saved' if saved else ''}", bar=bar,
           runner=run_saved if saved else None)


# ---- seeded random shapes (D, M, N, B, H and dtype drawn together) ------------------------------
def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.6 else "fp32"
        D = int(rng.choice([16, 32]))
        M = int(rng.choice([1, 17, 32, 33, 100, 128, 129, 256, 257, 400, 512]))
        N = int(rng.choice([1, 2, 63, 64, 65, 127, 128, 129, 255, 257, 1000, 3001]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        cases.append((i, dtype, D, M, N, B, H))
    return cases


@pytest.mark.parametrize("i,dtype,D,M,N,B,H", _random_cases(12, 4048))
def test_bwd_random_shapes(i, dtype, D, M, N, B, H):
    w = make_workload(1, B=B, H=H, N=N, M=M, D=D, dtype=dtype, kind="gauss", seed=8000 + i)
    _check(w, label=f"random {i}: {dtype} D={D} M={M} N={N} B={B} H={H}")


def _random_bf16_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([16, 32]))
        M = int(rng.choice([1, 31, 32, 64, 95, 200, 256, 300, 511, 512]))
        N = int(rng.choice([1, 31, 32, 33, 500, 1023, 4097, 20000]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        kind = str(rng.choice(["gauss", "cube"]))
        cases.append((i, D, M, N, B, H, kind))
    return cases


@pytest.mark.parametrize("i,D,M,N,B,H,kind", _random_bf16_cases(8, 5150))
def test_bwd_random_shapes_bf16(i, D, M, N, B, H, kind):
    # More seeded shapes for the bf16 kernels with fp16 operands (token encode and synthesis, the
    # decode call's latent side): ragged latent blocks, ragged token groups and stages, both widths.
    w = make_workload(1 if kind == "gauss" else 2, B=B, H=H, N=N, M=M, D=D, dtype="bf16", kind=kind,
                      seed=9100 + i)
    _check(w, label=f"random bf16 {i}: D={D} M={M} N={N} B={B} H={H} {kind}")


@pytest.mark.parametrize("dtype,N", [("fp32", 2), ("fp32", 3), ("bf16", 2), ("bf16", 3)])
def test_bwd_tiny_token_counts(dtype, N):
    """Two or three tokens against 257 latents, at the usual bars. A softmax row over two tokens
    has the cotangent P1 P2 (dP1 - dP2), which can be far below the row term c = <dZ, Z> (encode)
    or <G, Qd> (synthesis). Any error in c then dominates dQf and dQseed, so Z and Qd must come
    from P.V products as exact as the backward's own: with single-bf16 probabilities and values
    in the recompute, c was about 2^-8 off and these two tensors reached 3.6% of their RMS."""
    w = make_workload(1, B=1, H=1, N=N, M=257, D=16, dtype=dtype, kind="gauss", seed=8003)
    _check(w, label=f"bwd tiny N={N} {dtype}")


# ---- the backward from the forward's saved state (flarepp_mix_forward_saved, _backward_saved) ----
@pytest.mark.parametrize("cfg,kw", [(1, {}), (3, dict(B=2, H=2, N=3000)), (4, dict(B=1, H=2, N=20000)),
                                    (4, dict(B=1, H=2, N=3001, M=300, seed=9)), (5, dict(H=2, N=65536))])
def test_saved_forward_and_backward(cfg, kw):
    """flarepp_mix_forward_saved's output meets the forward's bar against the oracle, and
    flarepp_mix_backward_saved from its workspace meets the backward's bars against the oracle for
    two cotangents in a row (the backward only reads the saved state), and is bitwise the
    recomputing flarepp_mix_backward: the saved statistics are the ones that pass recomputes."""
    import rank_latent_routing_amd as fl
    from gpu_util import oracle_head
    w = make_workload(cfg, **kw)
    dt = 1 if w.dtype == "bf16" else 0
    say(f"[saved] {w.name} {kw}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}")
    dev = to_device(w)
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    need = fl.flarepp_backward_workspace_bytes(w.B, w.H, w.N, w.M, w.D, dt)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_ref = torch.empty(need, dtype=torch.uint8, device="cuda")
    Y = fl.flarepp_mix_forward_saved(*args, workspace=ws)
    torch.cuda.synchronize()
    Yn = Y.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            worst = max(worst, slice_err(Yn[b, h], oracle_head(w, b, h)["Y"], w.dtype))
    say(f"[saved] forward: worst {worst:.3g} (bar {tol(w.dtype)})")
    assert worst <= tol(w.dtype)
    for k, seed in enumerate((None, 77)):
        dY = make_cotangent(w, seed=seed)
        dy = _device(dY, w.dtype)
        a = fl.flarepp_mix_backward_saved(*args, dy, workspace=ws)
        b = fl.flarepp_mix_backward(*args, dy, workspace=ws_ref)
        torch.cuda.synchronize()
        a = {n: v.float().cpu().numpy().astype(np.float64) for n, v in a.items()}
        b = {n: v.float().cpu().numpy().astype(np.float64) for n, v in b.items()}
        ref = oracle_backward(w, dY)
        for n in a:
            assert np.array_equal(a[n], b[n]), (k, n)
        worst = {}
        for n in ("dK", "dV", "dS"):
            for bb in range(w.B):
                for h in range(w.H):
                    worst[n] = max(worst.get(n, 0.0), _err(a[n][bb, h], ref[n][bb, h], w.dtype))
        for n in ("dQseed", "dQf"):
            for h in range(w.H):
                worst[n] = max(worst.get(n, 0.0), _err(a[n][h], ref[n][h], w.dtype))
        worst["dg"] = float(np.max(np.abs(a["dg"] - ref["dg"]) / np.maximum(ref["dg_scale"], 1e-30)))
        say(f"[saved] backward {k}: worst {worst}")
        for n, e in worst.items():
            assert e <= tol(w.dtype), (k, n, e)
