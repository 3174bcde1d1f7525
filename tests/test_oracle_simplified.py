"""Pins of the oracle's simplified FLARE++ (Appendix A.8, Eq. 20; CPU only).

The simplified variant routes with the synthesized query alone, Q = SDPA(Qseed, Sk, Sv) with
separate synthesis values and no fixed query or gate, then encodes and decodes as in Eq. 8. The
pins: torch's SDPA composed the same way, the mixer it becomes when the mixer's fixed query is zero
and its gate one, and the closed form for constant synthesis values. Planted mistakes in the
oracle are each caught.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import flarepp_oracle as orc


def _case(seed=0, N=120, M=9, D=16):
    rng = np.random.default_rng(seed)
    return dict(K=rng.standard_normal((N, D)), V=rng.standard_normal((N, D)), Sk=rng.standard_normal((N, D)) * 1.5,
                Sv=rng.standard_normal((N, D)), Qseed=rng.standard_normal((M, D)))


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)[None, None]


def check_torch_composition(impl, seed=1, **kw):
    c = _case(seed, **kw)
    Qd = F.scaled_dot_product_attention(_t(c["Qseed"]), _t(c["Sk"]), _t(c["Sv"]))
    Z = F.scaled_dot_product_attention(Qd, _t(c["K"]), _t(c["V"]))
    Y = F.scaled_dot_product_attention(_t(c["K"]), Qd, Z)
    got = impl(c["K"], c["V"], c["Sk"], c["Sv"], c["Qseed"])
    return max(np.abs(got["Y"] - Y[0, 0].numpy()).max(), np.abs(got["Z"] - Z[0, 0].numpy()).max(),
               np.abs(got["Qd"] - Qd[0, 0].numpy()).max())


def check_mixer_relation(impl, seed=2):
    # The mixer with Qf = 0 (N0(0) = 0 with the epsilon inside the root) and g = 1 routes with
    # Qd = SDPA(Qseed, N0(S), N0(S)): the simplified variant with Sk = Sv = N0(S) (torch rms_norm).
    c = _case(seed)
    S = c["Sk"]
    Sn = F.rms_norm(torch.from_numpy(S), (S.shape[1],), eps=orc.RMS_EPS).numpy()
    got = impl(c["K"], c["V"], Sn, Sn, c["Qseed"])
    ref = oracle.mix_head(c["K"], c["V"], S, c["Qseed"], np.zeros_like(c["Qseed"]), 1.0)
    return np.abs(got["Y"] - ref["Y"]).max()


def check_constant_values(impl, seed=3):
    # Sv_n = s for every token: every synthesis softmax row averages s, so every routing query is s;
    # all latents then hold the same Z, and every token's output is softmax_n(s K^T / sqrt(D)) V.
    c = _case(seed)
    s = np.random.default_rng(seed + 100).standard_normal(c["K"].shape[1])
    Sv = np.broadcast_to(s, c["Sv"].shape).copy()
    got = impl(c["K"], c["V"], c["Sk"], Sv, c["Qseed"])
    D = c["K"].shape[1]
    w = np.exp(c["K"] @ s / np.sqrt(D))
    y = (w / w.sum()) @ c["V"]
    return max(np.abs(got["Qd"] - s).max(), np.abs(got["Y"] - y).max())


def _pins(impl):
    return (check_torch_composition(impl) < 1e-12 and check_torch_composition(impl, seed=4, N=77, M=5, D=32) < 1e-12
            and check_mixer_relation(impl) < 1e-12 and check_constant_values(impl) < 1e-12)


def test_matches_torch_sdpa_composition():
    assert check_torch_composition(oracle.simplified_mix_head) < 1e-12
    assert check_torch_composition(oracle.simplified_mix_head, seed=4, N=77, M=5, D=32) < 1e-12


def test_is_the_mixer_with_zero_fixed_query_and_unit_gate():
    assert check_mixer_relation(oracle.simplified_mix_head) < 1e-12


def test_constant_synthesis_values_closed_form():
    assert check_constant_values(oracle.simplified_mix_head) < 1e-12


def test_blocked_and_batched_forms_agree():
    c = _case(5, N=300)
    whole = oracle.simplified_mix_head(c["K"], c["V"], c["Sk"], c["Sv"], c["Qseed"])
    blocked = oracle.simplified_mix_head(c["K"], c["V"], c["Sk"], c["Sv"], c["Qseed"], block=64)
    assert np.abs(whole["Y"] - blocked["Y"]).max() < 1e-13
    b = oracle.simplified_mix(*(c[k][None, None] for k in ("K", "V", "Sk", "Sv")), c["Qseed"][None])
    assert np.abs(b["Y"][0, 0] - whole["Y"]).max() == 0.0


def _mut_shared_values(K, V, Sk, Sv, Qseed, block=None):
    return oracle.simplified_mix_head(K, V, Sk, Sk, Qseed)  # the keys reused as values


def _mut_normalized_keys(K, V, Sk, Sv, Qseed, block=None):
    return oracle.simplified_mix_head(K, V, orc.rms_normalize(Sk), Sv, Qseed)  # N0 on the given keys


def _mut_normalized_query(K, V, Sk, Sv, Qseed, block=None):
    Qd = orc.rms_normalize(orc.sdpa(Qseed, Sk, Sv))  # N0 on the synthesized query
    Z = orc.encode(Qd, K, V)
    return {"Qd": Qd, "Q": Qd, "Z": Z, "Y": orc.decode(K, Qd, Z)}


def _mut_seed_reference(K, V, Sk, Sv, Qseed, block=None):
    Qd = orc.sdpa(Qseed, Sk, Sv) + orc.rms_normalize(Qseed)  # a fixed reference added back
    Z = orc.encode(Qd, K, V)
    return {"Qd": Qd, "Q": Qd, "Z": Z, "Y": orc.decode(K, Qd, Z)}


@pytest.mark.parametrize("mutant", [_mut_shared_values, _mut_normalized_keys, _mut_normalized_query,
                                    _mut_seed_reference])
def test_planted_mistake_is_caught(mutant):
    assert _pins(oracle.simplified_mix_head)
    assert not _pins(mutant)
