"""GPU parity of the HIP mixer (through the C ABI) against the float64 oracle.

Bars (per (b, h) slice): fp32 max|Y - Y_ref| / max|Y_ref| <= 1e-5; bf16 inputs with fp32
accumulation max|Y - Y_ref| <= 2e-2 RMS(Y_ref). The latent stages Qd, Q, Z (exported in fp32 before
any cast) are held to the same bars.
"""
import numpy as np
import pytest

from gpu_util import oracle_head, run_gpu, say, slice_err, tol, to_device
from workloads import make_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_routing_amd as fl
    fl.lib()  # fails loudly when the library is missing


def _check(w, heads=None, block=None, stages=True, label="", bf16_storage=False):
    """bf16_storage: for bf16 outputs whose spread reaches several times their RMS, the per-element
    bar adds the representation error of the two bf16 tensors on the path to Y (Y itself, and the
    latents Z that decode reads), 2^-8 |Y_ref| together; the latent stages keep the plain bar."""
    say(f"[parity] {label or w.name}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D} {w.dtype}")
    Y, Qd, Q, Z = run_gpu(w, debug=True)
    assert np.isfinite(Y).all()
    worst = {}
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in pairs:
        ref = oracle_head(w, b, h, block=block)
        if bf16_storage:
            rms = np.sqrt(np.mean(ref["Y"] ** 2))
            excess = np.abs(Y[b, h] - ref["Y"]) - 2.0 ** -8 * np.abs(ref["Y"])
            errs = {"Y": max(float(excess.max()), 0.0) / rms}
        else:
            errs = {"Y": slice_err(Y[b, h], ref["Y"], w.dtype)}
        if stages:
            errs.update(Qd=slice_err(Qd[b, h], ref["Qd"], w.dtype), Q=slice_err(Q[b, h], ref["Q"], w.dtype),
                        Z=slice_err(Z[b, h], ref["Z"], w.dtype))
        for k, e in errs.items():
            worst[k] = max(worst.get(k, 0.0), e)
    say(f"[parity] {label or w.name}: worst {worst} (bar {tol(w.dtype)})")
    for k, e in worst.items():
        assert e <= tol(w.dtype), (k, e)
    return Y


def test_cfg1_fp32_full():
    _check(make_workload(1))


@pytest.mark.parametrize("N", [1, 31, 127, 128, 129, 1000, 3001])
def test_cfg1_shapes_fp32_ragged_tokens(N):
    _check(make_workload(1, N=N, seed=100 + N), label=f"cfg1 N={N}")


def test_cfg2_bf16_ragged():
    _check(make_workload(2, B=2, H=3, N=5000))


def test_cfg3_bf16_and_gate_zero_head():
    w = make_workload(3, B=2)
    Y = _check(w)
    # Head 0 has g = 0: the routing queries are N0(Qf) whatever S and Qseed hold, so the output
    # is bitwise unchanged when they change (Section 3.2: g -> 0 is fixed-query routing).
    w2 = make_workload(3, B=2)
    rng = np.random.default_rng(5)
    w2.S = (w.S ^ rng.integers(0, 4, size=w.S.shape, dtype=np.uint16)).astype(np.uint16)
    w2.Qseed = w.Qseed[:, ::-1].copy()
    Y2 = run_gpu(w2, debug=False)
    assert np.array_equal(Y[:, 0], Y2[:, 0])
    assert not np.array_equal(Y[:, 1], Y2[:, 1])


def test_cfg4_bf16_reduced():
    _check(make_workload(4, B=1, H=2, N=20000))


def test_cfg4_peaked_bf16_reduced():
    _check(make_workload(4, B=1, H=2, N=20000, peaked=True))


def test_cfg5_bf16_reduced():
    _check(make_workload(5, H=2, N=150000), block=32768)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [16, 32])
@pytest.mark.parametrize("M", [1, 17, 33, 100, 200, 512])
def test_latent_counts(dtype, D, M):
    # Ragged latent counts on the mesh-like input family.
    _check(make_workload(2, B=1, H=2, N=700, M=M, D=D, dtype=dtype, seed=7 * M + D), label=f"M={M} D={D} {dtype}")


@pytest.mark.parametrize("M", [257, 300, 480, 511])
def test_large_ragged_latent_counts(M):
    # bf16 D=32 with M > 256: one 16-wave workgroup per chunk (some waves without latents when
    # M < 512), 256-token stages with a partial last stage, and decode latent blocks of both
    # parities with a ragged last block.
    _check(make_workload(4, B=1, H=2, N=3001, M=M, seed=11 * M), label=f"M={M}")


@pytest.mark.parametrize("M", [17, 100])
def test_latent_counts_gaussian_inputs(M):
    _check(make_workload(3, B=1, H=2, N=700, M=M, seed=3 * M), label=f"gauss M={M}")


@pytest.fixture
def force_exact():
    import rank_latent_routing_amd as fl
    prev = fl.flarepp_debug_force_exact(True)
    yield
    fl.flarepp_debug_force_exact(prev)


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(B=1, H=3, N=5000)), (3, dict(B=1)),
                                    (4, dict(B=1, H=2, N=20000)), (5, dict(H=1, N=70000)),
                                    (2, dict(B=1, H=2, N=700, M=17, D=32, dtype="fp32"))])
def test_exact_path_everywhere(force_exact, cfg, kw):
    # The running-maximum softmaxes of all three calls, on well-conditioned inputs.
    _check(make_workload(cfg, **kw), label=f"exact cfg{cfg} {kw}")


def _decode_rows_out_of_range(w, b=0, h=0):
    """Fraction of tokens whose zero-shift decode row sum, sum_m 2^(log2(e) q_m.k/sqrt(D)), falls
    outside [2^-80, 2^100]: the tokens the library must recompute with running maxima."""
    import oracle
    K, S = w.f64("K")[b, h], w.f64("S")[b, h]
    Q = oracle.gate(w.f64("Qf")[h], oracle.synthesis(w.f64("Qseed")[h], S), float(w.g[h]))
    L = (K @ Q.T) * (np.log2(np.e) / np.sqrt(K.shape[1]))
    m = L.max(axis=1)
    lsum = m + np.log2(np.exp2(L - m[:, None]).sum(axis=1))
    return float(((lsum > 100.0) | (lsum < -80.0)).mean())


def test_wide_logits_take_the_exact_path():
    # Keys scaled x24: routing logits reach about 200 (log2 units), beyond the range the zero-shift
    # pass accepts, so encode chunks and decode tokens fall back to running maxima. The routing
    # logits stay accurate in bf16 runs (exact bf16 keys, hi/lo queries, fp32 accumulation).
    w = make_workload(3, B=1, H=2, N=3000, M=64, seed=11)
    from workloads.gen import _store
    w.K = _store(w.f64("K") * 24.0, "bf16")
    assert _decode_rows_out_of_range(w, 0, 0) > 0.05
    _check(w, label="wide logits")


# Seed and key scales: the seeds' learned scale sets the temperature of the synthesis logits
# (Appendix A.3, Eq. 14) and the routing keys' scale that of the routing logits (Appendix A.4), so
# logits of several tens (log2 units) are ordinary operating points. The grid covers the zero-shift
# window and, with the exact path forced, the running-maximum passes. The latent stages Qd, Q, Z
# (fp32 exports) keep the plain bar. In bf16 the outputs become one-hot picks of single latent rows
# as the scales grow, up to 15 times RMS(Y), and storing Y and Z in bf16 alone then costs more than
# 2% of RMS (tests/test_oracle.py::test_bf16_storage_of_heavy_tailed_outputs_exceeds_the_plain_bar),
# so Y takes the plain bar plus that storage rounding, 2^-8 |Y_ref| per element.
SCALE_GRID = [(1, 1), (2, 1), (3, 1), (4, 1), (5, 1), (6, 1), (1, 2), (1, 4), (1, 8), (1, 12), (3, 6), (4, 9),
              (6, 12)]


def _scaled(w, seeds, keys):
    from workloads.gen import _store
    w.Qseed = _store(w.f64("Qseed") * seeds, w.dtype)
    w.K = _store(w.f64("K") * keys, w.dtype)
    return w


@pytest.mark.parametrize("exact", [False, True], ids=["default", "exact"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seeds,keys", SCALE_GRID)
def test_seed_and_key_scale_sweep(seeds, keys, dtype, exact):
    import rank_latent_routing_amd as fl
    w = _scaled(make_workload(3, B=1, H=2, N=3000, M=64, dtype=dtype, seed=41 + 7 * seeds + keys), seeds, keys)
    prev = fl.flarepp_debug_force_exact(exact)
    try:
        _check(w, label=f"seeds x{seeds} keys x{keys} {dtype} {'exact' if exact else 'default'}",
               bf16_storage=(dtype == "bf16"))
    finally:
        fl.flarepp_debug_force_exact(prev)


@pytest.mark.parametrize("exact", [False, True], ids=["default", "exact"])
@pytest.mark.parametrize("seeds,keys", [(4, 1), (6, 1), (1, 8), (6, 12)])
def test_seed_and_key_scales_d16(seeds, keys, exact):
    # bf16 with D = 16 runs both passes on the 16x16x32 path (raw synthesis keys with a per-token
    # factor on the zero-shift pass too).
    import rank_latent_routing_amd as fl
    w = _scaled(make_workload(2, B=1, H=2, N=3000, M=48, seed=17 * seeds + keys), seeds, keys)
    prev = fl.flarepp_debug_force_exact(exact)
    try:
        _check(w, label=f"D=16 seeds x{seeds} keys x{keys} {'exact' if exact else 'default'}", bf16_storage=True)
    finally:
        fl.flarepp_debug_force_exact(prev)


@pytest.mark.parametrize("dtype,big", [("fp32", 36.0), ("bf16", 40.0)])
def test_zero_shift_and_exact_chunks_mixed(dtype, big):
    # Large keys in two token ranges: the chunks and decode token groups that hold them fall back
    # to the exact path, all others keep the zero-shift result.
    w = make_workload(4, B=1, H=2, N=20000, dtype=dtype)
    from workloads.gen import _store
    K = w.f64("K")
    K[:, :, 17000:17500] *= big
    K[:, :, 8000:8100] *= big
    w.K = _store(K, dtype)
    frac = _decode_rows_out_of_range(w, 0, 0)
    assert 0.0 < frac < 0.03
    # The decode rows of the large keys are one-hot picks of single latents, about 6 RMS(Y) in size:
    # in bf16 their own storage costs up to 1.2% of RMS, beyond what the plain bar leaves.
    _check(w, label=f"mixed {dtype}", bf16_storage=(dtype == "bf16"))


def test_gate_one_and_zero_everywhere():
    for gval in (0.0, 1.0):
        _check(make_workload(2, B=1, H=2, N=2000, g=gval), label=f"g={gval}")


def test_determinism_and_entry_points_agree():
    import rank_latent_routing_amd as fl
    w = make_workload(4, B=1, H=2, N=30000)
    dev = to_device(w)
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    a = fl.flarepp_mix(*args)
    b = fl.flarepp_mix_ws(*args)
    c, _, _, _ = fl.flarepp_mix_debug(*args)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_empty_problem():
    import rank_latent_routing_amd as fl
    K = torch.zeros((1, 2, 0, 16), dtype=torch.bfloat16, device="cuda")
    Qs = torch.zeros((2, 8, 16), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(2, dtype=torch.float32, device="cuda")
    out = fl.flarepp_mix(K, K, K, Qs, Qs, g)
    torch.cuda.synchronize()
    assert out.shape == K.shape


# ---------------------------------------------------------------- full sizes, sampled

def _full(cfg, heads, ntok=None, **kw):
    """The workload at its full size in the launch configuration the benchmark times, checked on the
    (b, h) slices `heads` ("all": every slice; the oracle runs them on a pool of host threads)."""
    w = make_workload(cfg, **kw)
    say(f"[full] {w.name}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D}")
    Y = run_gpu(w, debug=False)
    assert np.isfinite(Y).all()
    if heads == "all":
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rng = np.random.default_rng(cfg)
    picks = {bh: (None if ntok is None else rng.choice(w.N, size=ntok, replace=False)) for bh in heads}

    def err(bh):
        # (plain metric, bf16: the same beyond the storage rounding 2^-8 |Y_ref| of each element)
        b, h = bh
        ref = oracle_head(w, b, h, block=65536)["Y"]
        idx = picks[bh]
        got, want = (Y[b, h], ref) if idx is None else (Y[b, h][idx], ref[idx])
        if w.dtype == "fp32":
            e = slice_err(got, want, w.dtype)
            return e, e
        rms = np.sqrt(np.mean(ref ** 2))
        d = np.abs(got - want)
        return d.max() / rms, max(float((d - 2.0 ** -8 * np.abs(want)).max()), 0.0) / rms

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=8) as pool:
        errs = dict(zip(heads, pool.map(err, heads)))
    worst = max(errs, key=lambda k: errs[k][0])
    plain_ok = sum(e[0] <= tol(w.dtype) for e in errs.values())
    say(f"[full] {w.name}: {len(errs)} slices, worst {errs[worst][0]:.3g} at (b, h) = {worst} "
        f"({errs[worst][1]:.3g} beyond storage); {plain_ok} of {len(errs)} within the plain bar")
    # bf16 outputs are held to the plain bar beyond their storage rounding: in heavy-tailed slices
    # (max|Y| several times RMS(Y)) rounding Y to bf16 alone moves an element by up to 2^-8 |Y|.
    for bh, e in errs.items():
        assert e[1] <= tol(w.dtype), (bh, e)
    return w, Y


def test_full_cfg2():
    _full(2, "all")


def test_full_cfg3():
    _full(3, "all")


def test_full_cfg4_and_peaked():
    _full(4, "all")
    _full(4, [(0, 0), (1, 2), (1, 7)], peaked=True)


def test_full_cfg5_two_heads():
    _full(5, [(0, 3), (0, 6)])


def test_full_cfg5_constant_values_pass_through():
    # A row-stochastic operator maps a constant value field to itself (Eq. 4), at every token.
    w = make_workload(5)
    from workloads.gen import _store
    v = np.random.default_rng(3).standard_normal((w.H, w.D))
    w.V = _store(np.broadcast_to(v[None, :, None, :], (w.B, w.H, w.N, w.D)), "bf16")
    Y = run_gpu(w, debug=False)
    ref = w.f64("V")[:, :, :1, :]
    err = np.abs(Y - ref).max() / np.sqrt(np.mean(ref ** 2))
    say(f"[full] cfg5 constant V err {err:.3g}")
    assert err <= tol("bf16")


# ---- plain FLARE (Section 3.1, Eq. 3): fixed latent queries, no synthesis, no gate.
@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(B=2, H=3, N=5000)), (4, dict(B=1, H=2, N=20000)),
                                    (5, dict(H=1, N=70000)), (4, dict(B=1, H=2, N=3001, M=300, seed=9))])
def test_plain_flare(cfg, kw):
    import oracle
    import rank_latent_routing_amd as fl
    w = make_workload(cfg, **kw)
    say(f"[parity] flare cfg{cfg} {kw}")
    dev = to_device(w)
    Y = fl.flarepp_flare(dev["K"], dev["V"], dev["Qf"]).float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle.flare(w.f64("Qf")[h], w.f64("K")[b, h], w.f64("V")[b, h])
            worst = max(worst, slice_err(Y[b, h], ref, w.dtype))
    say(f"[parity] flare cfg{cfg}: worst {worst} (bar {tol(w.dtype)})")
    assert worst <= tol(w.dtype)


def test_plain_flare_full_cfg5_one_head():
    # The 1M-token workload at its full size through flarepp_flare; head 5 against the oracle in
    # token blocks.
    import oracle
    import rank_latent_routing_amd as fl
    w = make_workload(5)
    say(f"[full] flare {w.name}: B={w.B} H={w.H} N={w.N} M={w.M} D={w.D}")
    dev = to_device(w)
    Y = fl.flarepp_flare(dev["K"], dev["V"], dev["Qf"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y.float()).all())
    h = 5
    got = Y[0, h].float().cpu().numpy().astype(np.float64)
    from workloads import to_float64
    ref = oracle.flare(to_float64(w.Qf[h], w.dtype), to_float64(w.K[0, h], w.dtype), to_float64(w.V[0, h], w.dtype),
                       block=65536)
    err = slice_err(got, ref, w.dtype)
    say(f"[full] flare cfg5 head {h}: err {err:.3g} (bar {tol(w.dtype)})")
    assert err <= tol(w.dtype)


def test_plain_flare_equals_mixer_with_gate_zero():
    # g = 0 routes with N0(Qf) alone (Section 3.2), so the mixer equals FLARE on N0(Qf); the two
    # entry points share the encode and decode kernels.
    import rank_latent_routing_amd as fl
    w = make_workload(4, B=1, H=2, N=20000, g=0.0)
    dev = to_device(w)
    Y = fl.flarepp_mix(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    qf = dev["Qf"].float()
    qn = (qf / torch.sqrt((qf * qf).mean(dim=-1, keepdim=True) + 1e-6)).to(dev["Qf"].dtype).contiguous()
    Y2 = fl.flarepp_flare(dev["K"], dev["V"], qn)
    torch.cuda.synchronize()
    # N0(Qf) is rounded to bf16 here but kept in fp32 inside the gate, so compare to the bar.
    ref = Y.float().cpu().numpy().astype(np.float64)
    got = Y2.float().cpu().numpy().astype(np.float64)
    for h in range(w.H):
        assert slice_err(got[0, h], ref[0, h], w.dtype) <= tol(w.dtype)


# ---- seeded random shapes (D, M, N, B, H, dtype and the gate drawn together) ---------------------
def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.6 else "fp32"
        D = int(rng.choice([16, 32]))
        M = int(rng.choice([1, 2, 31, 32, 33, 64, 100, 127, 128, 129, 255, 256, 257, 300, 480, 512]))
        N = int(rng.choice([1, 2, 17, 63, 64, 65, 255, 256, 257, 999, 1024, 2500, 4097]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        cases.append((i, dtype, D, M, N, B, H))
    return cases


@pytest.mark.parametrize("i,dtype,D,M,N,B,H", _random_cases(16, 2024))
def test_random_shapes_forward(i, dtype, D, M, N, B, H):
    w = make_workload(1, B=B, H=H, N=N, M=M, D=D, dtype=dtype, kind="gauss", seed=7000 + i)
    _check(w, label=f"random {i}: {dtype} D={D} M={M} N={N} B={B} H={H}")
