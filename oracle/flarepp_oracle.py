"""Plain float64 CPU oracle of the FLARE++ mixer: its forward and backward passes, the plain-FLARE and
simplified variants, and the block around it (feature projections, per-head normalizations, gate
logit, output projection).

TEST INFRASTRUCTURE ONLY. This module is the reference against which the GPU library is checked.
Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may import it; the
mixer library never calls it and has no CPU fallback.

It evaluates the definitions of "FLARE++: Low-rank attention with attention-synthesized routing"
(arXiv 2608.11519 v2) literally, in numpy float64, and shares no code with the GPU path. Softmaxes
are two-pass (row maximum, then the normalized exponentials); the routing factors are formed
explicitly. The only blocking is over tokens when a factor would not fit in memory, and it keeps
the same two-pass definition (see ``sdpa_tokens``).

Readings where the pages leave a step open:
* RMS normalization N0 uses epsilon 1e-6 inside the square root (the pages state none).
* Qseed and K arrive already normalized by the caller (the learned-scale normalization N_a of
  Section 3.2 / Appendix A.3-A.4 is outside the mixer); N0 is applied to S and to Qf only.
* g is the gate value itself (the pages write g = sigmoid(gamma)).
* Decode normalizes over the M latents (softmax of the transposed scores, Section 3.1, Eq. 4).
* The block (``mixer_block``): projections are X W (+ b) with W [C_in, C_out] as the pages write
  them, biases optional (Appendix A.5 initializes them at zero); the per-head normalizations are RMS
  normalizations for every dtype, with epsilon 1e-6, N_a carrying one scale vector of D entries shared
  by the heads; the gate is sigmoid(gamma).
"""
from __future__ import annotations

import math

import numpy as np

#: Epsilon of the affine-free RMS normalization N0.
RMS_EPS = 1e-6


def rms_normalize(x: np.ndarray) -> np.ndarray:
    """N0: divide each row (last axis, the head width D) by its root-mean-square.

    Section 3.2 (definition of N0 next to Eq. 5) and Appendix A.4, Eq. 16: every row of N0(x) has
    unit RMS (up to the epsilon).
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + RMS_EPS)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, computed in two passes: subtract the row maximum, exponentiate,
    divide by the row sum. The shift is the identity of Appendix B.3, Eq. 29."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def sdpa(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Scaled dot-product attention, Section 3.1, Eq. 1: softmax(q k^T / sqrt(D)) v, with the
    softmax over the rows of k (the keys). q: [Nq, D], k: [Nk, D], v: [Nk, Dv]."""
    D = q.shape[-1]
    return softmax_rows(q @ k.T / math.sqrt(D)) @ v


def sdpa_tokens(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int) -> np.ndarray:
    """Eq. 1 for a short query set against a long key set, with the keys taken in blocks of
    ``block`` rows so that the [Nq, Nk] score matrix is never held whole. First pass: the row maxima
    over all keys. Second pass: the exponentials shifted by those maxima, summed and applied to v.
    Equal to ``sdpa`` up to summation order."""
    return sdpa_tokens_stats(q, k, v, block)[0]


def sdpa_tokens_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int):
    """``sdpa_tokens`` that also returns the softmax's row maxima and shifted row sums, so that
    P = exp(q k^T / sqrt(D) - max) / sum. Returns (o, row_max, den)."""
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D)
    n = k.shape[0]
    row_max = np.full(q.shape[0], -np.inf)
    for a in range(0, n, block):
        row_max = np.maximum(row_max, (q @ k[a:a + block].T * scale).max(axis=1))
    den = np.zeros(q.shape[0])
    num = np.zeros((q.shape[0], v.shape[1]))
    for a in range(0, n, block):
        e = np.exp(q @ k[a:a + block].T * scale - row_max[:, None])
        den += e.sum(axis=1)
        num += e @ v[a:a + block]
    return num / den[:, None], row_max, den


def synthesis(Qseed: np.ndarray, S: np.ndarray, block: int | None = None) -> np.ndarray:
    """Routing-query correction Qd (Section 3.2, Eq. 5-6; Appendix A.6, Eq. 19): the seeds attend
    over the N0-normalized synthesis keys, which are also the values. Qseed [M, D], S [N, D]."""
    keys = rms_normalize(S)
    if block is None:
        return sdpa(Qseed, keys, keys)
    return sdpa_tokens(Qseed, keys, keys, block)


def gate(Qf: np.ndarray, Qd: np.ndarray, g: float) -> np.ndarray:
    """Routing queries Q = N0(Qf) + g Qd (Section 3.2, Eq. 7; Appendix A.4, Eq. 15). Qd itself is
    not normalized (Appendix A.4, "Why the synthesized query is not normalized")."""
    return rms_normalize(Qf) + float(g) * np.asarray(Qd, dtype=np.float64)


def encode(Q: np.ndarray, K: np.ndarray, V: np.ndarray, block: int | None = None) -> np.ndarray:
    """Latent values Z = SDPA(Q, K, V) (Eq. 8, first call): softmax over the N tokens."""
    if block is None:
        return sdpa(Q, K, V)
    return sdpa_tokens(Q, K, V, block)


def decode(K: np.ndarray, Q: np.ndarray, Z: np.ndarray, block: int | None = None) -> np.ndarray:
    """Token outputs Y = SDPA(K, Q, Z) (Eq. 8, second call): the keys K act as queries against the
    M routing queries, softmax over the M latents. Rows are independent, so blocking over the
    query tokens changes nothing."""
    if block is None:
        return sdpa(K, Q, Z)
    return np.concatenate([sdpa(K[a:a + block], Q, Z) for a in range(0, K.shape[0], block)])


def mix_head(K, V, S, Qseed, Qf, g, block: int | None = None) -> dict:
    """One (batch, head) slice of the mixer, Appendix A.1, Eq. 11. Returns the stages
    ``Qd`` [M, D], ``Q`` [M, D], ``Z`` [M, D] and the output ``Y`` [N, D]."""
    Qd = synthesis(Qseed, S, block)
    Q = gate(Qf, Qd, g)
    Z = encode(Q, K, V, block)
    Y = decode(K, Q, Z, block)
    return {"Qd": Qd, "Q": Q, "Z": Z, "Y": Y}


def mix(K, V, S, Qseed, Qf, g, block: int | None = None) -> dict:
    """The mixer over all batch elements and heads. K, V, S: [B, H, N, D]; Qseed, Qf: [H, M, D]
    (shared over the batch); g: [H]. Returns stacked stages Qd, Q, Z [B, H, M, D] and Y [B, H, N, D]."""
    B, H = K.shape[:2]
    out = {"Qd": [], "Q": [], "Z": [], "Y": []}
    for b in range(B):
        rows = {key: [] for key in out}
        for h in range(H):
            r = mix_head(K[b, h], V[b, h], S[b, h], Qseed[h], Qf[h], g[h], block)
            for key in out:
                rows[key].append(r[key])
        for key in out:
            out[key].append(np.stack(rows[key]))
    return {key: np.stack(val) for key, val in out.items()}


# ---- Backward pass ------------------------------------------------------------------------------

def rms_normalize_backward(x: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """Cotangent of N0 (Section 3.2). With y = x r and r = (mean(x^2) + eps)^(-1/2) per row,
    dx = r dy - r^3 x mean(x dy) (the derivative of r is -r^3 x / D)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + RMS_EPS)
    return r * dy - r ** 3 * x * np.mean(x * dy, axis=-1, keepdims=True)


def sdpa_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray):
    """Cotangents of o = softmax(q k^T s) v, s = D^(-1/2), given dout (Appendix B.5, Eq. 46-49 on a
    single shard, whose log-normalizer gets no cotangent): with P the normalized probabilities and
    c_i = <dout_i, o_i>, dv = P^T dout, dS = P * (dout v^T - c), dq = s dS k, dk = s dS^T q.
    Returns (dq, dk, dv)."""
    s = 1.0 / math.sqrt(q.shape[-1])
    P = softmax_rows(q @ k.T * s)
    o = P @ v
    dout = np.asarray(dout, dtype=np.float64)
    dv = P.T @ dout
    c = np.sum(dout * o, axis=-1, keepdims=True)
    dS = P * (dout @ v.T - c)
    return s * dS @ k, s * dS.T @ q, dv


def mix_head_backward(K, V, S, Qseed, Qf, g, dY) -> dict:
    """Cotangents of one (batch, head) slice of the mixer (Appendix A.1, Eq. 11) given dY [N, D]:
    the decode call, then the encode call, the gate (Eq. 7) and the synthesis call, each SDPA by
    ``sdpa_backward`` and each N0 by ``rms_normalize_backward``. The decode's keys are the routing
    queries and its queries the token keys, so K and Q receive cotangents from both calls.
    Returns dK, dV, dS [N, D], dQseed, dQf [M, D] and dg (a scalar)."""
    Sn = rms_normalize(S)
    Qd = sdpa(Qseed, Sn, Sn)
    Q = gate(Qf, Qd, g)
    Z = sdpa(Q, K, V)
    dK_dec, dQ_dec, dZ = sdpa_backward(K, Q, Z, dY)
    dQ_enc, dK_enc, dV = sdpa_backward(Q, K, V, dZ)
    dQ = dQ_dec + dQ_enc
    dQseed, dSn_keys, dSn_values = sdpa_backward(Qseed, Sn, Sn, float(g) * dQ)
    return {"dK": dK_dec + dK_enc, "dV": dV, "dS": rms_normalize_backward(S, dSn_keys + dSn_values),
            "dQseed": dQseed, "dQf": rms_normalize_backward(Qf, dQ), "dg": float(np.sum(dQ * Qd)),
            "dQ": dQ, "dZ": dZ}


def sdpa_backward_tokens(q, k, v, fwd, dout, block: int):
    """``sdpa_backward`` for a short query set against a long key set (softmax over the keys, the
    tokens), with the keys taken in blocks of ``block`` rows so that no [Nq, Nk] factor is held
    whole (Appendix B.5, Eq. 46-49). ``fwd`` is the call's forward, (o, row_max, den) from
    ``sdpa_tokens_stats``: P = exp(q k^T s - row_max) / den, and c = <dout, o>. dq sums over the
    blocks, while dk and dv are per key row. Equal to ``sdpa_backward`` up to summation order.
    Returns (dq, dk, dv)."""
    s = 1.0 / math.sqrt(q.shape[-1])
    o, row_max, den = fwd
    dout = np.asarray(dout, dtype=np.float64)
    c = np.sum(dout * o, axis=-1, keepdims=True)
    dq = np.zeros(q.shape)
    dk = np.empty(k.shape)
    dv = np.empty((k.shape[0], dout.shape[1]))
    for a in range(0, k.shape[0], block):
        kb, vb = k[a:a + block], v[a:a + block]
        P = np.exp(q @ kb.T * s - row_max[:, None]) / den[:, None]
        dS = P * (dout @ vb.T - c)
        dq += s * dS @ kb
        dk[a:a + block] = s * dS.T @ q
        dv[a:a + block] = P.T @ dout
    return dq, dk, dv


def mix_head_backward_blocked(K, V, S, Qseed, Qf, g, dY, block: int) -> dict:
    """``mix_head_backward`` with the tokens taken in blocks of ``block`` rows, for token counts
    whose [N, M] factors would not fit in memory. The same calls in the same order: the decode call
    (rows independent: ``sdpa_backward`` per token block, its latent cotangents summed over the
    blocks), then the encode and synthesis calls by ``sdpa_backward_tokens``, the gate and the two
    N0's. Returns the same fields, and Qd."""
    K, V, S = (np.asarray(x, dtype=np.float64) for x in (K, V, S))
    dY = np.asarray(dY, dtype=np.float64)
    Sn = rms_normalize(S)
    syn = sdpa_tokens_stats(Qseed, Sn, Sn, block)
    Qd = syn[0]
    Q = gate(Qf, Qd, g)
    enc = sdpa_tokens_stats(Q, K, V, block)
    Z = enc[0]
    dK_dec = np.empty(K.shape)
    dQ_dec = np.zeros(Q.shape)
    dZ = np.zeros(Z.shape)
    for a in range(0, K.shape[0], block):
        dq, dk, dv = sdpa_backward(K[a:a + block], Q, Z, dY[a:a + block])
        dK_dec[a:a + block] = dq
        dQ_dec += dk
        dZ += dv
    dQ_enc, dK_enc, dV = sdpa_backward_tokens(Q, K, V, enc, dZ, block)
    dQ = dQ_dec + dQ_enc
    dQseed, dSn_keys, dSn_values = sdpa_backward_tokens(Qseed, Sn, Sn, syn, float(g) * dQ, block)
    return {"dK": dK_dec + dK_enc, "dV": dV, "dS": rms_normalize_backward(S, dSn_keys + dSn_values),
            "dQseed": dQseed, "dQf": rms_normalize_backward(Qf, dQ), "dg": float(np.sum(dQ * Qd)),
            "dQ": dQ, "dZ": dZ, "Qd": Qd}


def mix_backward(K, V, S, Qseed, Qf, g, dY) -> dict:
    """``mix_head_backward`` over all batch elements and heads. The seeds, Qf and g are shared over
    the batch, so their cotangents are summed over it. Returns dK, dV, dS [B, H, N, D], dQseed,
    dQf [H, M, D] and dg [H]."""
    B, H = K.shape[:2]
    out = {"dK": np.zeros(K.shape), "dV": np.zeros(K.shape), "dS": np.zeros(K.shape),
           "dQseed": np.zeros(Qseed.shape), "dQf": np.zeros(Qf.shape), "dg": np.zeros(H)}
    for b in range(B):
        for h in range(H):
            r = mix_head_backward(K[b, h], V[b, h], S[b, h], Qseed[h], Qf[h], g[h], dY[b, h])
            out["dK"][b, h], out["dV"][b, h], out["dS"][b, h] = r["dK"], r["dV"], r["dS"]
            out["dQseed"][h] += r["dQseed"]
            out["dQf"][h] += r["dQf"]
            out["dg"][h] += r["dg"]
    return out


def routing_factors(Q: np.ndarray, K: np.ndarray):
    """The two routing factors of Section 3.1, Eq. 3-4, for queries Q [M, D] and keys K [N, D]:
    W_enc = softmax(S) [M, N] (over tokens) and W_dec = softmax(S^T) [N, M] (over latents), with
    S = Q K^T / sqrt(D)."""
    Sc = Q @ K.T / math.sqrt(Q.shape[-1])
    return softmax_rows(Sc), softmax_rows(Sc.T)


def mixing_matrix(Q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """The N x N operator W_eff = W_dec W_enc of Eq. 4 / Eq. 9 (rank <= M). Small N only."""
    W_enc, W_dec = routing_factors(Q, K)
    return W_dec @ W_enc


def flare(Q: np.ndarray, K: np.ndarray, V: np.ndarray, block: int | None = None) -> np.ndarray:
    """Fixed-query FLARE, Section 3.1, Eq. 3: Z = SDPA(Q, K, V), Y = SDPA(K, Q, Z) (tokens in blocks
    of ``block`` rows when given)."""
    return decode(K, Q, encode(Q, K, V, block), block)


def simplified_mix_head(K, V, Sk, Sv, Qseed, block: int | None = None) -> dict:
    """One (batch, head) slice of simplified FLARE++ (Appendix A.8, Eq. 20): the routing queries are
    the synthesized correction alone, Q = Qd = SDPA(Qseed, Sk, Sv), with no fixed query, no gate and
    separate synthesis values; then Z = SDPA(Q, K, V) and Y = SDPA(K, Q, Z) as in Eq. 8. The learned
    scales of Qseed and Sk are the caller's (as for the mixer's Qseed and K), so the keys Sk and values
    Sv are used as given. Returns ``Qd`` (= ``Q``), ``Z`` and ``Y``."""
    Qd = sdpa(Qseed, Sk, Sv) if block is None else sdpa_tokens(Qseed, Sk, Sv, block)
    Z = encode(Qd, K, V, block)
    Y = decode(K, Qd, Z, block)
    return {"Qd": Qd, "Q": Qd, "Z": Z, "Y": Y}


def simplified_mix(K, V, Sk, Sv, Qseed, block: int | None = None) -> dict:
    """``simplified_mix_head`` over all batch elements and heads (Qseed [H, M, D] shared over the
    batch). Returns stacked Qd, Z [B, H, M, D] and Y [B, H, N, D]."""
    B, H = K.shape[:2]
    out = {"Qd": [], "Z": [], "Y": []}
    for b in range(B):
        rows = {key: [] for key in out}
        for h in range(H):
            r = simplified_mix_head(K[b, h], V[b, h], Sk[b, h], Sv[b, h], Qseed[h], block)
            for key in out:
                rows[key].append(r[key])
        for key in out:
            out[key].append(np.stack(rows[key]))
    return {key: np.stack(val) for key, val in out.items()}


def encode_sharded(Q: np.ndarray, K: np.ndarray, V: np.ndarray, bounds) -> tuple:
    """The token-sharded encoder of Appendix B.2-B.3: each shard r (token range bounds[r]) gives
    its local log-normalizer L_r (Eq. 25) and local output Z_r (Eq. 26); the stable schedule of
    Eq. 30-33 merges them: L_max = max_r L_r, d_r = exp(L_r - L_max), U_r = d_r Z_r, d = sum d_r,
    U = sum U_r, Z = U / d, L = L_max + log d. An empty shard returns L_r = -inf and Z_r = 0
    (Appendix B.3). Returns (Z, L)."""
    s = 1.0 / math.sqrt(Q.shape[-1])
    Ls, Zs = [], []
    for a, b in bounds:
        if b <= a:
            Ls.append(np.full(Q.shape[0], -np.inf))
            Zs.append(np.zeros((Q.shape[0], V.shape[1])))
            continue
        Sr = s * Q @ K[a:b].T
        m = Sr.max(axis=1)
        Ls.append(m + np.log(np.exp(Sr - m[:, None]).sum(axis=1)))
        Zs.append(softmax_rows(Sr) @ V[a:b])
    L_max = np.max(np.stack(Ls), axis=0)
    d_r = [np.exp(L - L_max) for L in Ls]
    d = np.sum(d_r, axis=0)
    U = np.sum([dr[:, None] * Zr for dr, Zr in zip(d_r, Zs)], axis=0)
    return U / d[:, None], L_max + np.log(d)


# ---- The block around the mixer: feature projections, per-head normalizations, output projection --

def rms_normalize_scaled(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """N_a: RMS normalization over the head width with a learned per-channel scale (Section 3.2, where
    N_a and N0 are introduced; Appendix C.2 names its places: the synthesis seeds and the routing keys).
    One scale vector of D entries serves every head (Appendix A.7: a per-head normalization carries D
    parameters)."""
    return rms_normalize(x) * np.asarray(scale, dtype=np.float64)


def split_heads(T: np.ndarray, H: int) -> np.ndarray:
    """[B, N, C] -> [B, H, N, D], D = C / H: head h owns channels h D .. h D + D - 1 (Section 3.1,
    "Full self-attention": the projections split into H heads of width D = C / H)."""
    B, N, C = T.shape
    return np.ascontiguousarray(T.reshape(B, N, H, C // H).transpose(0, 2, 1, 3))


def merge_heads(Y: np.ndarray) -> np.ndarray:
    """[B, H, N, D] -> [B, N, H D]: the head outputs concatenated along the channels (Section 3.1, "Full self-attention")."""
    B, H, N, D = Y.shape
    return np.ascontiguousarray(Y.transpose(0, 2, 1, 3).reshape(B, N, H * D))


def linear(X: np.ndarray, W: np.ndarray, b: np.ndarray | None = None) -> np.ndarray:
    """X W (+ b): a pointwise projection with W [C_in, C_out], as the pages write it."""
    y = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64)
    return y if b is None else y + np.asarray(b, dtype=np.float64)


def project(X, Wk, Wv, Ws, H, nk, bk=None, bv=None, bs=None):
    """The projections in front of the mixer for X [B, N, C]: routing keys K = N_a(X W_K) (Section 3.2,
    before Eq. 8), values V = X W_V, and synthesis keys S = X W~_K (Eq. 5, which the mixer normalizes
    with N0 itself). Returns K, V, S as [B, H, N, D]."""
    K = rms_normalize_scaled(split_heads(linear(X, Wk, bk), H), nk)
    V = split_heads(linear(X, Wv, bv), H)
    S = split_heads(linear(X, Ws, bs), H)
    return K, V, S


def out_project(Y, Wo, bo=None):
    """The output projection: heads concatenated, then W_O (Section 3.1, "Full self-attention").
    Y [B, H, N, D] -> [B, N, C]."""
    return linear(merge_heads(Y), Wo, bo)


def sigmoid(x):
    """The logistic function; the gate is g = sigmoid(gamma) (Section 3.2, Eq. 7)."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def mixer_block(X, Wk, Wv, Ws, Wo, Qseed, Qf, gamma, nq, nk, bk=None, bv=None, bs=None, bo=None,
                block: int | None = None) -> dict:
    """The mixer with its projections (Section 3.2, Eq. 5-8; Appendix A.6-A.7, C.2), then the output
    projection: K, V, S from ``project``; synthesis seeds N_a(Qseed) with scale nq; g = sigmoid(gamma);
    the mixer (``mix``) on them; out = concat_h(Y_h) W_O. X [B, N, C]; W_* [C, C] (X W); Qseed, Qf
    [H, M, D]; gamma [H]; nq, nk [D]. Returns K, V, S, Y [B, H, N, D] and ``out`` [B, N, C]."""
    H = Qseed.shape[0]
    K, V, S = project(X, Wk, Wv, Ws, H, nk, bk, bv, bs)
    r = mix(K, V, S, rms_normalize_scaled(Qseed, nq), Qf, sigmoid(gamma), block)
    return {"K": K, "V": V, "S": S, "Y": r["Y"], "out": out_project(r["Y"], Wo, bo)}
