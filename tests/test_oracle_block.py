"""Pins of the oracle's mixer block: the projections in front of the mixer, the per-head
normalizations, the gate logit and the output projection (Section 3.2, Eq. 5-8; Appendix A.5-A.7,
C.2; Section 3.1, "Full self-attention", for the head split and the output projection). CPU only.

The pins:
* torch's own primitives (matmul, rms_norm with and without weight, sigmoid, SDPA), one (batch,
  head) at a time over the heads' channel ranges, in float64;
* the near-identity initialization of Appendix A.5 at Delta W = 0 (W = I, no bias): the keys are the
  input's head slices, RMS-normalized, written out with explicit loops;
* every routing-key row has the RMS of the key scale (N_a), whatever the input;
* a joint permutation of the heads (projection columns, output-projection rows, seeds, fixed queries,
  gate logits) leaves the block's output unchanged;
* the output projection is affine in Y.
Planted mistakes in the oracle (head split order, a missing or misplaced normalization, the gate
logit used as the gate, a dropped bias, a transposed weight) each fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import flarepp_oracle as orc


def _case(seed=0, B=2, N=60, H=2, D=16, M=5):
    rng = np.random.default_rng(seed)
    C = H * D
    W = lambda: rng.standard_normal((C, C)) / math.sqrt(C)
    return dict(X=rng.standard_normal((B, N, C)), Wk=W(), Wv=W(), Ws=W(), Wo=W(),
                bk=rng.standard_normal(C) * 0.1, bv=rng.standard_normal(C) * 0.1,
                bs=rng.standard_normal(C) * 0.1, bo=rng.standard_normal(C) * 0.1,
                Qseed=rng.standard_normal((H, M, D)), Qf=rng.standard_normal((H, M, D)),
                gamma=rng.standard_normal(H), nq=1.0 + 0.3 * rng.standard_normal(D),
                nk=1.0 + 0.3 * rng.standard_normal(D))


def _run(impl, c):
    return impl(c["X"], c["Wk"], c["Wv"], c["Ws"], c["Wo"], c["Qseed"], c["Qf"], c["gamma"], c["nq"],
                c["nk"], c["bk"], c["bv"], c["bs"], c["bo"])


def _torch_block(c):
    """The block from torch float64 library calls, one (batch, head) at a time: the projections as
    X W + b (torch.matmul), head h as the channel range h D .. h D + D - 1 (Section 3.1, "Full
    self-attention"), N_a and N0 by torch's rms_norm (Section 3.2; Appendix C.2), the gate
    g_h = sigmoid(gamma_h) (Eq. 7), the mixer of Eq. 5-8 with torch's scaled_dot_product_attention
    per call, and the outputs of all heads written back into their channel ranges before W_O."""
    as_t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    X = as_t(c["X"])
    n_heads, _, width = c["Qseed"].shape
    unit_rms = lambda x: F.rms_norm(x, (width,), eps=orc.RMS_EPS)
    scaled_rms = lambda x, w: F.rms_norm(x, (width,), weight=as_t(w), eps=orc.RMS_EPS)
    attend = lambda q, k, v: F.scaled_dot_product_attention(q[None], k[None], v[None])[0]
    keys_all = X @ as_t(c["Wk"]) + as_t(c["bk"])
    values_all = X @ as_t(c["Wv"]) + as_t(c["bv"])
    syn_all = X @ as_t(c["Ws"]) + as_t(c["bs"])
    K = torch.empty(X.shape[0], n_heads, X.shape[1], width, dtype=torch.float64)
    V = torch.empty_like(K)
    Y = torch.empty_like(K)
    merged = torch.empty_like(X)
    for b in range(X.shape[0]):
        for h in range(n_heads):
            cols = slice(h * width, (h + 1) * width)
            K[b, h] = scaled_rms(keys_all[b, :, cols], c["nk"])
            V[b, h] = values_all[b, :, cols]
            syn = unit_rms(syn_all[b, :, cols])
            correction = attend(scaled_rms(as_t(c["Qseed"][h]), c["nq"]), syn, syn)
            gate_h = torch.sigmoid(as_t(c["gamma"][h]))
            routing = unit_rms(as_t(c["Qf"][h])) + gate_h * correction
            latents = attend(routing, K[b, h], V[b, h])
            Y[b, h] = attend(K[b, h], routing, latents)
            merged[b, :, cols] = Y[b, h]
    out = merged @ as_t(c["Wo"]) + as_t(c["bo"])
    return {"K": K.numpy(), "V": V.numpy(), "Y": Y.numpy(), "out": out.numpy()}


def check_torch_composition(impl, seed=1, **kw):
    c = _case(seed, **kw)
    got, ref = _run(impl, c), _torch_block(c)
    return max(np.abs(got[k] - ref[k]).max() / np.abs(ref[k]).max() for k in ref)


def check_identity_projection(impl, seed=2):
    # Appendix A.5 at Delta W = 0: W = I and zero biases, so K_h = N_a(X_h), V_h = X_h, S_h = X_h.
    c = _case(seed, B=1, N=7, H=2, D=16, M=3)
    C = c["X"].shape[-1]
    c.update(Wk=np.eye(C), Wv=np.eye(C), Ws=np.eye(C), bk=np.zeros(C), bv=np.zeros(C), bs=np.zeros(C),
             nk=np.ones(16))
    got = _run(impl, c)
    X = c["X"]
    err = 0.0
    for n in range(7):
        for h in range(2):
            row = [X[0, n, h * 16 + d] for d in range(16)]
            r = math.sqrt(sum(v * v for v in row) / 16 + orc.RMS_EPS)
            for d in range(16):
                err = max(err, abs(got["K"][0, h, n, d] - row[d] / r), abs(got["V"][0, h, n, d] - row[d]))
    return err


def check_key_rms(impl, seed=3):
    # N_a(x) = N0(x) * scale: with the scale divided out every routing-key row has unit RMS, up to
    # the epsilon inside the root (about 5e-7 for rows of RMS near 1).
    c = _case(seed)
    K = _run(impl, c)["K"] / c["nk"]
    rms = np.sqrt(np.mean(K * K, axis=-1))
    return np.abs(rms - 1.0).max()


def check_head_permutation(impl, seed=4):
    c = _case(seed, H=3, D=16)
    base = _run(impl, c)["out"]
    perm = np.array([2, 0, 1])
    D = 16
    cols = np.concatenate([np.arange(p * D, p * D + D) for p in perm])
    p = dict(c)
    for k in ("Wk", "Wv", "Ws"):
        p[k] = c[k][:, cols]
    for k in ("bk", "bv", "bs"):
        p[k] = c[k][cols]
    p["Wo"] = c["Wo"][cols, :]
    for k in ("Qseed", "Qf", "gamma"):
        p[k] = c[k][perm]
    return np.abs(_run(impl, p)["out"] - base).max() / np.abs(base).max()


def _pins(impl):
    return (check_torch_composition(impl) < 1e-12 and check_torch_composition(impl, seed=5, H=4, D=32, N=33) < 1e-12
            and check_identity_projection(impl) < 1e-12 and check_key_rms(impl) < 1e-5
            and check_head_permutation(impl) < 1e-12)


def test_matches_torch_per_head_composition():
    assert check_torch_composition(oracle.mixer_block) < 1e-12
    assert check_torch_composition(oracle.mixer_block, seed=5, H=4, D=32, N=33) < 1e-12


def test_identity_projections_closed_form():
    assert check_identity_projection(oracle.mixer_block) < 1e-12


def test_routing_keys_have_the_scale_rms():
    assert check_key_rms(oracle.mixer_block) < 1e-5


def test_joint_head_permutation_leaves_output_unchanged():
    assert check_head_permutation(oracle.mixer_block) < 1e-12


def test_out_projection_is_affine_in_y():
    rng = np.random.default_rng(6)
    Y1, Y2 = rng.standard_normal((2, 2, 2, 9, 16))
    Wo, bo = rng.standard_normal((32, 32)), rng.standard_normal(32)
    lhs = oracle.out_project(2.0 * Y1 - 3.0 * Y2, Wo)
    assert np.abs(lhs - (2.0 * oracle.out_project(Y1, Wo) - 3.0 * oracle.out_project(Y2, Wo))).max() < 1e-12
    assert np.abs(oracle.out_project(Y1, Wo, bo) - oracle.out_project(Y1, Wo) - bo).max() < 1e-12


def test_split_and_merge_are_inverse():
    X = np.random.default_rng(7).standard_normal((2, 5, 48))
    assert np.array_equal(oracle.merge_heads(oracle.split_heads(X, 3)), X)
    assert np.array_equal(oracle.split_heads(X, 3)[1, 2, 4], X[1, 4, 32:48])


# ---- planted mistakes ---------------------------------------------------------------------------

def _block_with(project=None, seeds=None, gate=None, out=None):
    def impl(X, Wk, Wv, Ws, Wo, Qseed, Qf, gamma, nq, nk, bk=None, bv=None, bs=None, bo=None):
        H = Qseed.shape[0]
        K, V, S = (project or orc.project)(X, Wk, Wv, Ws, H, nk, bk, bv, bs)
        Qs = (seeds or orc.rms_normalize_scaled)(Qseed, nq)
        r = orc.mix(K, V, S, Qs, Qf, (gate or orc.sigmoid)(gamma))
        return {"K": K, "V": V, "S": S, "Y": r["Y"], "out": (out or orc.out_project)(r["Y"], Wo, bo)}
    return impl


def _split_dh(T, H):  # channels read as d H + h instead of h D + d
    B, N, C = T.shape
    return np.ascontiguousarray(T.reshape(B, N, C // H, H).transpose(0, 3, 1, 2))


def _project_split_dh(X, Wk, Wv, Ws, H, nk, bk=None, bv=None, bs=None):
    K = orc.rms_normalize_scaled(_split_dh(orc.linear(X, Wk, bk), H), nk)
    return K, _split_dh(orc.linear(X, Wv, bv), H), _split_dh(orc.linear(X, Ws, bs), H)


def _project_norm_v(X, Wk, Wv, Ws, H, nk, bk=None, bv=None, bs=None):
    K, V, S = orc.project(X, Wk, Wv, Ws, H, nk, bk, bv, bs)
    return K, orc.rms_normalize(V), S


def _project_no_scale(X, Wk, Wv, Ws, H, nk, bk=None, bv=None, bs=None):
    return orc.project(X, Wk, Wv, Ws, H, np.ones_like(nk), bk, bv, bs)


def _project_no_bias(X, Wk, Wv, Ws, H, nk, bk=None, bv=None, bs=None):
    return orc.project(X, Wk, Wv, Ws, H, nk, None, bv, bs)


def _project_transposed(X, Wk, Wv, Ws, H, nk, bk=None, bv=None, bs=None):
    return orc.project(X, Wk.T, Wv, Ws, H, nk, bk, bv, bs)


def _out_merge_dh(Y, Wo, bo=None):
    B, H, N, D = Y.shape
    return orc.linear(Y.transpose(0, 2, 3, 1).reshape(B, N, H * D), Wo, bo)


MUTANTS = {
    "split_dh": _block_with(project=_project_split_dh),
    "norm_on_values": _block_with(project=_project_norm_v),
    "key_scale_dropped": _block_with(project=_project_no_scale),
    "key_bias_dropped": _block_with(project=_project_no_bias),
    "key_weight_transposed": _block_with(project=_project_transposed),
    "seed_scale_dropped": _block_with(seeds=lambda Q, nq: orc.rms_normalize(Q)),
    "gate_logit_as_gate": _block_with(gate=lambda gamma: np.asarray(gamma, dtype=np.float64)),
    "merge_dh": _block_with(out=_out_merge_dh),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    assert _pins(oracle.mixer_block)
    assert not _pins(MUTANTS[name])
