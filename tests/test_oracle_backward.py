"""Pins of the oracle's backward pass (CPU only).

The oracle's cotangents are checked against torch autograd in float64 through a forward pass
written independently with torch ops (rms_norm, scaled_dot_product_attention), against central
finite differences of <Y, dY>, and against cotangents that the pages' definitions force to zero.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _inputs(seed, N=40, M=6, D=8, scale=1.0):
    rng = np.random.default_rng(seed)
    return dict(K=rng.standard_normal((N, D)) * scale, V=rng.standard_normal((N, D)), S=rng.standard_normal((N, D)),
                Qseed=rng.standard_normal((M, D)), Qf=rng.standard_normal((M, D)), g=float(rng.uniform(0.2, 0.9)),
                dY=rng.standard_normal((N, D)))


def _torch_forward(K, V, S, Qseed, Qf, g):
    # Section 3.2 Eq. 5-8 written with torch primitives (float64, CPU).
    D = K.shape[-1]
    n0 = lambda x: F.rms_norm(x, (D,), eps=oracle.RMS_EPS)
    Sn = n0(S)
    Qd = F.scaled_dot_product_attention(Qseed[None], Sn[None], Sn[None])[0]
    Q = n0(Qf) + g * Qd
    Z = F.scaled_dot_product_attention(Q[None], K[None], V[None])[0]
    return F.scaled_dot_product_attention(K[None], Q[None], Z[None])[0]


def test_backward_matches_torch_autograd():
    for seed in range(3):
        x = _inputs(seed)
        t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in x.items() if k not in ("g", "dY")}
        g = torch.tensor(x["g"], dtype=torch.float64, requires_grad=True)
        Y = _torch_forward(t["K"], t["V"], t["S"], t["Qseed"], t["Qf"], g)
        Y.backward(torch.tensor(x["dY"]))
        r = oracle.mix_head_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], x["dY"])
        for name in ("K", "V", "S", "Qseed", "Qf"):
            np.testing.assert_allclose(r["d" + name], t[name].grad.numpy(), rtol=1e-9, atol=1e-11)
        assert abs(r["dg"] - g.grad.item()) <= 1e-9 * max(1.0, abs(g.grad.item()))


def test_backward_matches_finite_differences():
    x = _inputs(7, N=24, M=5, D=8)
    r = oracle.mix_head_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], x["dY"])
    f = lambda y: float(np.sum(oracle.mix_head(y["K"], y["V"], y["S"], y["Qseed"], y["Qf"], y["g"])["Y"] * x["dY"]))
    rng = np.random.default_rng(1)
    h = 1e-5
    for name in ("K", "V", "S", "Qseed", "Qf"):
        d = rng.standard_normal(x[name].shape)
        xp, xm = dict(x), dict(x)
        xp[name], xm[name] = x[name] + h * d, x[name] - h * d
        fd = (f(xp) - f(xm)) / (2 * h)
        an = float(np.sum(r["d" + name] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    xp, xm = dict(x), dict(x)
    xp["g"], xm["g"] = x["g"] + h, x["g"] - h
    assert abs((f(xp) - f(xm)) / (2 * h) - r["dg"]) <= 1e-6 * max(1.0, abs(r["dg"]))


def test_gate_zero_cuts_the_synthesis_branch():
    # g = 0: the routing queries are N0(Qf) (Section 3.2), so S and the seeds get no cotangent.
    x = _inputs(3)
    r = oracle.mix_head_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], 0.0, x["dY"])
    assert np.all(r["dS"] == 0.0) and np.all(r["dQseed"] == 0.0)
    assert np.abs(r["dQf"]).max() > 0 and r["dg"] != 0.0


def test_constant_values_cut_every_routing_cotangent():
    # Row-stochastic routing (Section 3.1, Eq. 4) passes a constant V through unchanged, so the
    # output depends on V alone: every routing input has a zero cotangent.
    x = _inputs(4)
    x["V"] = np.tile(np.random.default_rng(0).standard_normal(x["V"].shape[1]), (x["V"].shape[0], 1))
    r = oracle.mix_head_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], x["dY"])
    for name in ("dK", "dS", "dQseed", "dQf"):
        assert np.abs(r[name]).max() <= 1e-12, name
    assert abs(r["dg"]) <= 1e-12
    # ...and V's cotangent is the column sums of the mixing matrix times dY: each row sum over tokens
    # of dV equals the sum of dY (the mixing matrix is row-stochastic).
    np.testing.assert_allclose(r["dV"].sum(axis=0), x["dY"].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_backward_is_linear_in_the_output_cotangent():
    x = _inputs(5)
    a = oracle.mix_head_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], x["dY"])
    b = oracle.mix_head_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], -2.5 * x["dY"])
    for name in ("dK", "dV", "dS", "dQseed", "dQf"):
        np.testing.assert_allclose(b[name], -2.5 * a[name], rtol=1e-12, atol=1e-13)


def test_batched_backward_sums_shared_parameters():
    rng = np.random.default_rng(9)
    B, H, N, M, D = 2, 2, 16, 4, 8
    K, V, S, dY = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    Qseed, Qf = rng.standard_normal((H, M, D)), rng.standard_normal((H, M, D))
    g = rng.uniform(0, 1, H)
    r = oracle.mix_backward(K, V, S, Qseed, Qf, g, dY)
    for h in range(H):
        parts = [oracle.mix_head_backward(K[b, h], V[b, h], S[b, h], Qseed[h], Qf[h], g[h], dY[b, h]) for b in range(B)]
        np.testing.assert_allclose(r["dQseed"][h], sum(p["dQseed"] for p in parts), rtol=1e-13)
        assert abs(r["dg"][h] - sum(p["dg"] for p in parts)) <= 1e-12


@pytest.mark.parametrize("mutant", ["no_c_term", "no_scale", "n0_no_cubic"])
def test_planted_backward_mistake_is_caught(monkeypatch, mutant):
    import oracle.flarepp_oracle as O
    orig_sdpa_bwd, orig_n0_bwd = O.sdpa_backward, O.rms_normalize_backward

    def bad_sdpa_backward(q, k, v, dout):
        s = 1.0 / math.sqrt(q.shape[-1])
        P = O.softmax_rows(q @ k.T * s)
        o = P @ v
        c = 0.0 if mutant == "no_c_term" else np.sum(dout * o, axis=-1, keepdims=True)
        dS = P * (dout @ v.T - c)
        t = 1.0 if mutant == "no_scale" else s
        return t * dS @ k, t * dS.T @ q, P.T @ dout

    def bad_n0_backward(x, dy):
        r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + O.RMS_EPS)
        return r * dy

    if mutant == "n0_no_cubic":
        monkeypatch.setattr(O, "rms_normalize_backward", bad_n0_backward)
    else:
        monkeypatch.setattr(O, "sdpa_backward", bad_sdpa_backward)
    with pytest.raises(AssertionError):
        test_backward_matches_torch_autograd()


# ---- The token-blocked backward (for token counts whose [N, M] factors do not fit in memory) ----

@pytest.mark.parametrize("N,block", [(3001, 512), (257, 64), (100, 1000)])
def test_blocked_backward_equals_whole(N, block):
    x = _inputs(20 + N, N=N, M=17, D=16)
    a = oracle.mix_head_backward(**x)
    b = oracle.mix_head_backward_blocked(**x, block=block)
    for k in a:
        ref = np.asarray(a[k])
        assert np.abs(np.asarray(b[k]) - ref).max() <= 1e-12 * np.abs(ref).max(), k


def test_blocked_backward_matches_torch_autograd():
    # Pinned on its own, not only through the whole-token oracle: autograd through the torch forward.
    x = _inputs(31, N=300, M=9, D=16)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in x.items() if k not in ("g", "dY")}
    g = torch.tensor(x["g"], dtype=torch.float64, requires_grad=True)
    Y = _torch_forward(t["K"], t["V"], t["S"], t["Qseed"], t["Qf"], g)
    (Y * torch.tensor(x["dY"])).sum().backward()
    r = oracle.mix_head_backward_blocked(**x, block=64)
    for k, ref in (("dK", t["K"].grad), ("dV", t["V"].grad), ("dS", t["S"].grad), ("dQseed", t["Qseed"].grad),
                   ("dQf", t["Qf"].grad)):
        np.testing.assert_allclose(r[k], ref.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)
    assert abs(r["dg"] - g.grad.item()) <= 1e-10 * max(1.0, abs(g.grad.item()))


def test_token_blocked_sdpa_backward_equals_whole():
    rng = np.random.default_rng(5)
    q, k, v, do = rng.standard_normal((7, 8)), rng.standard_normal((203, 8)), rng.standard_normal((203, 8)), \
        rng.standard_normal((7, 8))
    fwd = oracle.sdpa_tokens_stats(q, k, v, 50)
    np.testing.assert_allclose(fwd[0], oracle.sdpa(q, k, v), rtol=1e-13)
    for got, ref in zip(oracle.sdpa_backward_tokens(q, k, v, fwd, do, 50), oracle.sdpa_backward(q, k, v, do)):
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
