"""Pins of the float64 oracle against what the FLARE++ pages and the mathematics fix.

Each pin is independent of the oracle's own code path: a library routine evaluating the same
definition (torch's scaled_dot_product_attention and rms_norm, scipy's softmax), a closed form, an
invariant stated on the pages, or a brute-force evaluation through the explicit N x N operator.
The mutation tests at the end plant plausible mistakes in the oracle and check that the pins
catch each one.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import flarepp_oracle as orc
from workloads import make_workload


def _case(seed=0, N=64, M=8, D=16, g=None):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((N, D))
    V = rng.standard_normal((N, D))
    S = rng.standard_normal((N, D))
    Qseed = rng.standard_normal((M, D))
    Qf = rng.standard_normal((M, D))
    gv = rng.random() if g is None else g
    return K, V, S, Qseed, Qf, gv


# ---------------------------------------------------------------- library cross-checks

def _torch_mixer(K, V, S, Qseed, Qf, g):
    """One head of the mixer from torch float64 library calls, in the routing-factor form of
    Section 3.1 (Eq. 3-4) rather than the oracle's: the synthesis call (Eq. 5-6) through torch's
    scaled_dot_product_attention on the rms_norm-ed synthesis rows (keys and values at once), the
    gate blend of Eq. 7, then the encode and decode factors W_enc = softmax over tokens and
    W_dec = softmax over latents of one score matrix (Eq. 8), applied as Y = W_dec (W_enc V)."""
    as_t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    width = K.shape[-1]
    unit_rms = lambda x: F.rms_norm(x, (width,), eps=orc.RMS_EPS)
    syn_rows = unit_rms(as_t(S))
    correction = F.scaled_dot_product_attention(as_t(Qseed)[None], syn_rows[None], syn_rows[None])[0]
    routing = unit_rms(as_t(Qf)) + g * correction
    scores = routing @ as_t(K).T / math.sqrt(width)  # [M, N]
    w_enc = torch.softmax(scores, dim=1)
    w_dec = torch.softmax(scores.T, dim=1)
    latents = w_enc @ as_t(V)
    return {"Qd": correction.numpy(), "Q": routing.numpy(), "Z": latents.numpy(), "Y": (w_dec @ latents).numpy()}


def check_library(seed=1, N=200, M=12, D=16):
    K, V, S, Qseed, Qf, g = _case(seed, N, M, D)
    ref = _torch_mixer(K, V, S, Qseed, Qf, g)
    got = orc.mix_head(K, V, S, Qseed, Qf, g)
    return max(np.abs(got[k] - ref[k]).max() for k in ref)


def test_rms_normalize_matches_torch_rms_norm():
    x = np.random.default_rng(3).standard_normal((50, 32)) * 3
    ref = F.rms_norm(torch.from_numpy(x), (32,), eps=orc.RMS_EPS).numpy()
    assert np.abs(orc.rms_normalize(x) - ref).max() < 1e-13


def test_softmax_rows_matches_scipy():
    x = np.random.default_rng(4).standard_normal((7, 300)) * 20
    assert np.abs(orc.softmax_rows(x) - scipy.special.softmax(x, axis=-1)).max() < 1e-15


def test_sdpa_matches_torch():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((9, 32)), rng.standard_normal((100, 32)), rng.standard_normal((100, 32))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a)[None] for a in (q, k, v)))[0].numpy()
    assert np.abs(orc.sdpa(q, k, v) - ref).max() < 1e-13


def test_mixer_matches_torch_sdpa_composition():
    assert check_library() < 1e-12
    assert check_library(seed=2, N=97, M=5, D=32) < 1e-12


# ---------------------------------------------------------------- invariants the pages state

def check_row_stochastic(seed=6, N=300, M=16, D=16):
    K, V, S, Qseed, Qf, g = _case(seed, N, M, D)
    r = orc.mix_head(K, V, S, Qseed, Qf, g)
    W_enc, W_dec = orc.routing_factors(r["Q"], K)
    A_syn, _ = orc.routing_factors(Qseed, orc.rms_normalize(S))
    errs = [np.abs(W.sum(axis=1) - 1).max() for W in (W_enc, W_dec, A_syn)]
    negs = [W.min() for W in (W_enc, W_dec, A_syn)]
    return max(errs), min(negs), W_enc.shape, W_dec.shape


def test_softmax_factors_are_row_stochastic():
    err, neg, se, sd = check_row_stochastic()
    assert err < 1e-13 and neg >= 0
    assert se == (16, 300) and sd == (300, 16)  # W_enc over tokens, W_dec over latents


def check_rank(seed=7, N=256, M=8, D=16):
    K, V, S, Qseed, Qf, g = _case(seed, N, M, D)
    r = orc.mix_head(K, V, S, Qseed, Qf, g)
    sv = np.linalg.svd(orc.mixing_matrix(r["Q"], K), compute_uv=False)
    return sv[M] / sv[0], sv[M - 1] / sv[0]


def test_mixing_matrix_rank_at_most_M():
    ratio_after, ratio_at = check_rank()
    assert ratio_after < 1e-12
    assert ratio_at > 1e-10  # generic inputs reach rank M


def test_mixing_matrix_rank_cfg1_inputs():
    w = make_workload(1)
    K, V, S = w.f64("K")[0, 0], w.f64("V")[0, 0], w.f64("S")[0, 0]
    r = orc.mix_head(K, V, S, w.f64("Qseed")[0], w.f64("Qf")[0], w.g[0])
    Weff = orc.mixing_matrix(r["Q"], K)
    sv = np.linalg.svd(Weff, compute_uv=False)
    assert sv[w.M] / sv[0] < 1e-12
    # Brute force through the explicit N x N operator (Eq. 4 / Eq. 9) agrees with the factored path.
    assert np.abs(Weff @ V - r["Y"]).max() < 1e-12


def _bruteforce_loops(K, V, S, Qseed, Qf, g):
    """Scalar-loop evaluation through the explicit N x N mixing matrix (tiny inputs only)."""
    N, D = K.shape
    M = Qseed.shape[0]
    sc = 1.0 / math.sqrt(D)

    def n0(row):
        ms = sum(x * x for x in row) / len(row)
        return [x / math.sqrt(ms + orc.RMS_EPS) for x in row]

    def dot(a, b):
        return sum(x * y for x, y in zip(a, b))

    sk = [n0(list(S[n])) for n in range(N)]
    Qd = []
    for m in range(M):
        logits = [dot(Qseed[m], sk[n]) * sc for n in range(N)]
        top = max(logits)
        w = [math.exp(x - top) for x in logits]
        tot = sum(w)
        Qd.append([sum(w[n] * sk[n][d] for n in range(N)) / tot for d in range(D)])
    qf = [n0(list(Qf[m])) for m in range(M)]
    Q = [[qf[m][d] + g * Qd[m][d] for d in range(D)] for m in range(M)]
    Wenc = []
    for m in range(M):
        logits = [dot(Q[m], K[n]) * sc for n in range(N)]
        top = max(logits)
        w = [math.exp(x - top) for x in logits]
        tot = sum(w)
        Wenc.append([x / tot for x in w])
    Wdec = []
    for n in range(N):
        logits = [dot(K[n], Q[m]) * sc for m in range(M)]
        top = max(logits)
        w = [math.exp(x - top) for x in logits]
        tot = sum(w)
        Wdec.append([x / tot for x in w])
    Weff = [[sum(Wdec[n][m] * Wenc[m][j] for m in range(M)) for j in range(N)] for n in range(N)]
    return np.array([[sum(Weff[n][j] * V[j][d] for j in range(N)) for d in range(D)] for n in range(N)])


def test_bruteforce_scalar_loops():
    for seed, (N, M, D) in enumerate([(12, 3, 4), (9, 1, 2), (16, 5, 16)]):
        K, V, S, Qseed, Qf, g = _case(10 + seed, N, M, D)
        ref = _bruteforce_loops(K, V, S, Qseed, Qf, g)
        assert np.abs(orc.mix_head(K, V, S, Qseed, Qf, g)["Y"] - ref).max() < 1e-12


def check_g_zero(seed=8, N=150, M=10, D=16):
    K, V, S, Qseed, Qf, _ = _case(seed, N, M, D)
    y0 = orc.mix_head(K, V, S, Qseed, Qf, 0.0)["Y"]
    y_flare = orc.flare(orc.rms_normalize(Qf), K, V)
    rng = np.random.default_rng(seed + 100)
    y_pert = orc.mix_head(K, V, rng.standard_normal(S.shape), rng.standard_normal(Qseed.shape), Qf, 0.0)["Y"]
    return np.abs(y0 - y_flare).max(), np.abs(y0 - y_pert).max()


def test_gate_zero_is_fixed_query_flare():
    a, b = check_g_zero()
    assert a < 1e-13 and b < 1e-13


def check_rms_bounds(seed=9, N=400, M=32, D=16):
    worst_qd, worst_lo, worst_hi = 0.0, 1e9, -1e9
    for gval in (0.0, 0.3, 0.56, 1.0):
        K, V, S, Qseed, Qf, _ = _case(seed, N, M, D)
        r = orc.mix_head(K, V, S * 7.0, Qseed * 3.0, Qf, gval)
        rms_qd = np.sqrt(np.mean(r["Qd"] ** 2, axis=1))
        rms_q = np.sqrt(np.mean(r["Q"] ** 2, axis=1))
        # RMS of N0(Qf_m) is sqrt(ms / (ms + eps)), slightly below 1 because of the epsilon.
        ms_f = np.mean(Qf ** 2, axis=1)
        rms_f = np.sqrt(ms_f / (ms_f + orc.RMS_EPS))
        worst_qd = max(worst_qd, rms_qd.max())
        worst_lo = min(worst_lo, (rms_q - (rms_f - gval)).min())
        worst_hi = max(worst_hi, (rms_q - (1 + gval)).max())
    return worst_qd, worst_lo, worst_hi


def test_rms_bounds_of_synthesized_and_routing_queries():
    qd, lo, hi = check_rms_bounds()
    assert qd <= 1.0 + 1e-12          # Eq. 17: convex combination of unit-RMS rows
    assert lo >= -1e-12 and hi <= 1e-12  # 1 - g <= RMS(Q_m) <= 1 + g (lower end: RMS of N0(Qf_m))


def test_equal_synthesis_rows_make_the_bound_tight():
    K, V, S, Qseed, Qf, g = _case(11, 50, 6, 16)
    S[:] = S[0]
    Qd = orc.synthesis(Qseed, S)
    assert np.abs(Qd - orc.rms_normalize(S[:1])).max() < 1e-14
    assert abs(np.sqrt(np.mean(Qd ** 2, axis=1)).max() - 1.0) < 1e-6


def check_closed_forms(seed=12, N=120, M=7, D=16):
    K, V, S, Qseed, Qf, g = _case(seed, N, M, D)
    # M = 1: the decode softmax over one latent is 1, every token receives Z.
    r1 = orc.mix_head(K, V, S, Qseed[:1], Qf[:1], g)
    e_m1 = np.abs(r1["Y"] - r1["Z"][0]).max()
    # K = 0: both routing softmaxes are uniform, every token receives the mean of V.
    r0 = orc.mix_head(np.zeros_like(K), V, S, Qseed, Qf, g)
    e_k0 = np.abs(r0["Y"] - V.mean(axis=0)).max()
    # Constant V: W_eff is row-stochastic, so Y = V.
    vc = np.tile(V[:1], (N, 1))
    e_vc = np.abs(orc.mix_head(K, vc, S, Qseed, Qf, g)["Y"] - vc).max()
    return e_m1, e_k0, e_vc


def test_closed_forms():
    for e in check_closed_forms():
        assert e < 1e-13


def check_linearity_and_permutation(seed=13, N=90, M=6, D=16):
    K, V, S, Qseed, Qf, g = _case(seed, N, M, D)
    V2 = np.random.default_rng(seed + 1).standard_normal(V.shape)
    y = lambda v: orc.mix_head(K, v, S, Qseed, Qf, g)["Y"]
    e_lin = np.abs(y(2.0 * V - 3.0 * V2) - (2.0 * y(V) - 3.0 * y(V2))).max()
    perm = np.random.default_rng(seed + 2).permutation(N)
    ra = orc.mix_head(K, V, S, Qseed, Qf, g)
    rb = orc.mix_head(K[perm], V[perm], S[perm], Qseed, Qf, g)
    e_perm = max(np.abs(rb["Y"] - ra["Y"][perm]).max(), np.abs(rb["Z"] - ra["Z"]).max(),
                 np.abs(rb["Q"] - ra["Q"]).max())
    return e_lin, e_perm


def test_linear_in_V_and_permutation_equivariant():
    e_lin, e_perm = check_linearity_and_permutation()
    assert e_lin < 1e-12 and e_perm < 1e-13


def test_blocked_evaluation_equals_whole():
    K, V, S, Qseed, Qf, g = _case(14, 1000, 16, 32)
    a = orc.mix_head(K, V, S, Qseed, Qf, g)
    b = orc.mix_head(K, V, S, Qseed, Qf, g, block=77)
    for key in a:
        assert np.abs(a[key] - b[key]).max() < 1e-13
    assert np.abs(orc.flare(Qf, K, V) - orc.flare(Qf, K, V, block=77)).max() < 1e-13


def test_sharded_lse_merge_is_exact():
    K, V, S, Qseed, Qf, g = _case(15, 500, 10, 16)
    Q = orc.gate(Qf, orc.synthesis(Qseed, S), g)
    ref = orc.encode(Q * 5.0, K, V)  # a wide logit range
    for bounds in ([(0, 500)], [(0, 100), (100, 101), (101, 500)], [(0, 250), (250, 250), (250, 500)]):
        Z, L = orc.encode_sharded(Q * 5.0, K, V, bounds)
        assert np.abs(Z - ref).max() < 1e-13
        Sc = 5.0 * Q @ K.T / 4.0
        assert np.abs(L - scipy.special.logsumexp(Sc, axis=1)).max() < 1e-12


def test_peaked_logits_stay_finite():
    K, V, S, Qseed, Qf, g = _case(16, 64, 4, 16)
    r = orc.mix_head(K * 200.0, V, S, Qseed * 200.0, Qf, g)
    assert all(np.isfinite(r[k]).all() for k in r)


# ---------------------------------------------------------------- the input generator

def test_generator_bf16_cast_is_round_to_nearest_even():
    from workloads import bf16_bits_from_float, float_from_bf16_bits
    x = np.random.default_rng(17).standard_normal(10000).astype(np.float32) * 10
    x[:4] = [1.00390625, 1.01171875, -2.0078125, 3.0]  # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_float(x), ref)
    assert np.array_equal(float_from_bf16_bits(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_shaped():
    a = make_workload(2, N=300, B=2, H=3)
    b = make_workload(2, N=300, B=2, H=3)
    assert a.K.shape == (2, 3, 300, 16) and a.Qseed.shape == (3, 64, 16) and a.g.shape == (3,)
    assert a.K.dtype == np.uint16 and np.array_equal(a.K, b.K) and np.array_equal(a.S, b.S)
    c = make_workload(3, N=64, B=1)
    assert c.g[0] == 0.0 and c.K.shape == (1, 8, 64, 32)
    p = make_workload(4, N=128, B=1, H=2, peaked=True)
    q = make_workload(4, N=128, B=1, H=2)
    assert np.allclose(p.f64("K"), 4.0 * q.f64("K"), rtol=1e-2)
    s = make_workload(5, N=4096, H=2)
    assert s.K.shape == (1, 2, 4096, 32) and np.isfinite(s.f64("V")).all()


# ---------------------------------------------------------------- planted mistakes

def _all_pins_pass():
    ok = check_library() < 1e-12
    err, neg, se, sd = check_row_stochastic()
    ok &= err < 1e-13 and neg >= 0 and se[0] < se[1]
    ok &= check_rank()[0] < 1e-12
    a, b = check_g_zero()
    ok &= a < 1e-13 and b < 1e-13
    qd, lo, hi = check_rms_bounds()
    ok &= qd <= 1 + 1e-12 and lo >= -1e-12 and hi <= 1e-12
    ok &= all(e < 1e-13 for e in check_closed_forms())
    e_lin, e_perm = check_linearity_and_permutation()
    ok &= e_lin < 1e-12 and e_perm < 1e-13
    return bool(ok)


def _mut_decode_over_tokens(K, Q, Z, block=None):
    W = orc.softmax_rows((Q @ K.T / math.sqrt(K.shape[1]))).T  # normalizes over tokens, not latents
    return W @ Z


def _mut_no_scale(q, k, v):
    return orc.softmax_rows(q @ k.T) @ v


def _mut_unnormalized_values(Qseed, S, block=None):
    return orc.sdpa(Qseed, orc.rms_normalize(S), S)


def _mut_gate_sign(Qf, Qd, g):
    return orc.rms_normalize(Qf) - g * Qd


def _mut_normalized_qd(Qf, Qd, g):
    return orc.rms_normalize(Qf) + g * orc.rms_normalize(Qd)


def _mut_no_shift(s):
    e = np.exp(np.asarray(s) - 1.0)
    return e / e.sum(axis=-1, keepdims=True) * 0.999


def _mut_transposed_encode(Q, K, V, block=None):
    return orc.softmax_rows(K @ Q.T / math.sqrt(Q.shape[1])).T @ V * (Q.shape[0] / K.shape[0])


def _mut_eps(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-2)


@pytest.mark.parametrize("target,mutant", [
    ("decode", _mut_decode_over_tokens),
    ("sdpa", _mut_no_scale),
    ("synthesis", _mut_unnormalized_values),
    ("gate", _mut_gate_sign),
    ("gate", _mut_normalized_qd),
    ("softmax_rows", _mut_no_shift),
    ("encode", _mut_transposed_encode),
    ("rms_normalize", _mut_eps),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    assert _all_pins_pass()
    monkeypatch.setattr(orc, target, mutant)
    assert not _all_pins_pass()


def test_bf16_storage_of_heavy_tailed_outputs_exceeds_the_plain_bar():
    # The bar of the bf16 parity tests at large key scales, derived: with the routing keys scaled x2
    # (Gaussian inputs, M = 64; the sweep's seeds x1, keys x2 case, head 1) the decode rows become
    # near one-hot picks of single latent rows and max|Y| reaches 15 RMS(Y). Rounding the oracle's
    # own exact Y to bf16 (the output dtype) then moves it by more than the plain bar of 2e-2 RMS(Y),
    # so no bf16-output implementation can meet that bar there. Round to nearest moves each element
    # by at most the unit roundoff of bf16's 8-bit significand, 2^-8 |Y|, which is the per-element
    # allowance the tests add for such outputs.
    from workloads.gen import _store, to_float64
    w = make_workload(3, B=1, H=2, N=3000, M=64, dtype="bf16", seed=50)
    K = to_float64(_store(w.f64("K")[0, 1] * 2.0, "bf16"), "bf16")
    r = orc.mix_head(K, w.f64("V")[0, 1], w.f64("S")[0, 1], w.f64("Qseed")[1], w.f64("Qf")[1], float(w.g[1]))
    Y = r["Y"]
    rms = np.sqrt(np.mean(Y * Y))
    Yb = to_float64(_store(Y, "bf16"), "bf16")
    assert np.abs(Y).max() > 10 * rms
    assert np.abs(Yb - Y).max() > 3e-2 * rms
    assert (np.abs(Yb - Y) <= 2.0 ** -8 * np.abs(Y) * (1 + 1e-12)).all()
