"""Seeded synthetic workloads for the FLARE++ mixer.

Every tensor is drawn in float64 from ``numpy.random.Generator(PCG64(seed))`` and cast once to its
storage dtype with round-to-nearest-even. The cast tensors are the canonical inputs: the GPU path
receives their bits and the oracle receives their exact float64 values.

Shapes follow the mixer's interface: K, V, S are [B, H, N, D] (S holds the synthesis keys before
their RMS normalization), Qseed and Qf are [H, M, D] and shared over the batch, g is [H] float32
(the gate value in [0, 1]).

Input families (the source pages give no generator, so these are readings of the workload
descriptions; the pages evaluate on PDE meshes, DrivAerML surfaces and Long Range Arena, and these
synthetic families only stand in for their shapes and value ranges):

* ``gauss``   - K, V, S, Qseed, Qf i.i.d. N(0, 1); g ~ U[0, 1].
* ``cube``    - mesh-like smooth fields: N points uniform in the unit cube per batch element,
  features phi(x) = [x, y, z, sin(k_1.x), ..., sin(k_8.x)] with k_j ~ N(0, 4 I_3), and for each of
  K, V, S and each head a projection W in R^{11 x D} with N(0, 1/11) entries (shared over the batch).
* ``surface`` - the same features on points of a random closed star-shaped surface,
  r(u) = 1 + sum_{j<=4} a_j sin(w_j.u + p_j), a_j ~ U[0, 0.1], w_j ~ N(0, 9 I_3), p_j ~ U[0, 2 pi),
  x = r(u) u with u uniform on the sphere, rescaled per axis to the unit box.

``peaked`` multiplies K by 4 before the cast (a wider logit range for the softmaxes).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

#: The five workload shapes. ``kind`` selects the input family above.
CONFIGS = {
    1: dict(B=1, H=2, N=1024, M=32, D=16, dtype="fp32", kind="gauss"),
    2: dict(B=4, H=8, N=16384, M=64, D=16, dtype="bf16", kind="cube"),
    3: dict(B=32, H=8, N=4096, M=128, D=32, dtype="bf16", kind="gauss", g0_zero=True),
    4: dict(B=2, H=8, N=65536, M=256, D=32, dtype="bf16", kind="cube"),
    5: dict(B=1, H=8, N=1048576, M=512, D=32, dtype="bf16", kind="surface"),
}

#: What each workload stands for (its sizes are in CONFIGS).
DESCRIPTIONS = {
    1: "small fp32 case, Gaussian inputs",
    2: "mesh-like fields on points in the unit cube",
    3: "sequence-classification batch, Gaussian inputs, one head with gate 0",
    4: "mesh-like fields on 65536 points in the unit cube",
    5: "a million points on a random closed surface with mesh-like fields",
}

#: Input families as written in a benchmark record.
FAMILIES = {
    "gauss": "K, V, S i.i.d. N(0, 1)",
    "cube": "points uniform in the unit cube, sinusoidal-feature K/V/S",
    "surface": "points on a random closed surface, sinusoidal-feature K/V/S",
}

_SEED_BASE = 2608_11519


def workload_seed(cfg: int) -> int:
    """Seed of a configuration's draw (the peaked variant reuses its base configuration's seed)."""
    return _SEED_BASE + int(cfg)


def bf16_bits_from_float(x: np.ndarray) -> np.ndarray:
    """Round float values to bfloat16 (nearest, ties to even) and return the uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    # Finite values never carry out of 32 bits here (largest finite magnitude 0xFF7FFFFF + 0x8000).
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def float_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_float64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor (float32 array or bfloat16 bits)."""
    if dtype == "bf16":
        return float_from_bf16_bits(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_from_float(x)
    return np.ascontiguousarray(x, dtype=np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic mixer input. K, V, S, Qseed, Qf are stored tensors (float32, or uint16 bf16 bits)."""
    name: str
    B: int
    H: int
    N: int
    M: int
    D: int
    dtype: str
    K: np.ndarray
    V: np.ndarray
    S: np.ndarray
    Qseed: np.ndarray
    Qf: np.ndarray
    g: np.ndarray
    kind: str = "gauss"

    def f64(self, field: str) -> np.ndarray:
        """Exact float64 values of one stored tensor."""
        if field == "g":
            return self.g.astype(np.float64)
        return to_float64(getattr(self, field), self.dtype)


def _sphere_surface_points(rng: np.random.Generator, n: int) -> np.ndarray:
    z = rng.standard_normal((n, 3))
    u = z / np.linalg.norm(z, axis=1, keepdims=True)
    a = rng.uniform(0.0, 0.1, size=4)
    w = rng.normal(0.0, 3.0, size=(4, 3))
    p = rng.uniform(0.0, 2.0 * math.pi, size=4)
    r = 1.0 + np.sin(u @ w.T + p) @ a
    x = r[:, None] * u
    lo, hi = x.min(axis=0), x.max(axis=0)
    return (x - lo) / np.where(hi > lo, hi - lo, 1.0)


def make_workload(cfg: int, *, B: int | None = None, H: int | None = None, N: int | None = None,
                  M: int | None = None, D: int | None = None, dtype: str | None = None,
                  kind: str | None = None, peaked: bool = False, seed: int | None = None,
                  g: np.ndarray | float | None = None) -> Workload:
    """Draw configuration ``cfg``'s workload, optionally with some sizes overridden.

    The draw order is fixed: points and frequencies (mesh kinds) or K, V, S (gauss), then the
    projections (mesh kinds), then Qseed, Qf, g. Overriding a size changes the draw.
    """
    c = dict(CONFIGS[cfg])
    B = c["B"] if B is None else B
    H = c["H"] if H is None else H
    N = c["N"] if N is None else N
    M = c["M"] if M is None else M
    D = c["D"] if D is None else D
    dtype = c["dtype"] if dtype is None else dtype
    kind = c["kind"] if kind is None else kind
    rng = np.random.Generator(np.random.PCG64(workload_seed(cfg) if seed is None else seed))

    if kind == "gauss":
        Kf = rng.standard_normal((B, H, N, D))
        Vf = rng.standard_normal((B, H, N, D))
        Sf = rng.standard_normal((B, H, N, D))
        if peaked:
            Kf *= 4.0
        K, V, S = _store(Kf, dtype), _store(Vf, dtype), _store(Sf, dtype)
        del Kf, Vf, Sf
    elif kind in ("cube", "surface"):
        if kind == "cube":
            pts = rng.random((B, N, 3))
        else:
            pts = np.stack([_sphere_surface_points(rng, N) for _ in range(B)])
        freqs = rng.normal(0.0, 2.0, size=(8, 3))
        proj = rng.standard_normal((3, H, 11, D)) / math.sqrt(11.0)
        store_dt = np.uint16 if dtype == "bf16" else np.float32
        K = np.empty((B, H, N, D), store_dt)
        V = np.empty((B, H, N, D), store_dt)
        S = np.empty((B, H, N, D), store_dt)
        for b in range(B):
            feat = np.concatenate([pts[b], np.sin(pts[b] @ freqs.T)], axis=1)  # [N, 11]
            for h in range(H):
                k = feat @ proj[0, h]
                if peaked:
                    k *= 4.0
                K[b, h] = _store(k, dtype)
                V[b, h] = _store(feat @ proj[1, h], dtype)
                S[b, h] = _store(feat @ proj[2, h], dtype)
    else:
        raise ValueError(f"unknown input family {kind!r}")

    Qseed = _store(rng.standard_normal((H, M, D)), dtype)
    Qf = _store(rng.standard_normal((H, M, D)), dtype)
    gv = rng.random(H).astype(np.float32)
    if c.get("g0_zero"):
        gv[0] = 0.0
    if g is not None:
        gv = np.broadcast_to(np.asarray(g, dtype=np.float32), (H,)).copy()
    name = f"cfg{cfg}" + ("-peaked" if peaked else "")
    return Workload(name, B, H, N, M, D, dtype, K, V, S, Qseed, Qf, gv, kind)


def make_cotangent(w: Workload, seed: int | None = None) -> np.ndarray:
    """Seeded output cotangent dY for a workload: i.i.d. N(0, 1) of Y's shape [B, H, N, D], cast
    to the workload's storage dtype like the inputs."""
    rng = np.random.Generator(np.random.PCG64(workload_seed(0) + 7919 if seed is None else seed))
    return _store(rng.standard_normal((w.B, w.H, w.N, w.D)), w.dtype)


def make_synthesis_values(w: Workload, seed: int | None = None) -> np.ndarray:
    """Seeded separate synthesis values (the simplified variant's Sv) for a workload: i.i.d. N(0, 1)
    of shape [B, H, N, D], cast to the workload's storage dtype like the inputs."""
    rng = np.random.Generator(np.random.PCG64(workload_seed(0) + 104729 if seed is None else seed))
    return _store(rng.standard_normal((w.B, w.H, w.N, w.D)), w.dtype)


@dataclasses.dataclass
class BlockInputs:
    """Inputs of the mixer block around a workload: X [B, N, C] (C = H D), the projection matrices
    Wk, Wv, Ws, Wo [C, C] in the pages' orientation (the block computes X W), biases bk, bv, bs, bo [C],
    the key and seed scales nk, nq [D] (stored like the tensors), and the gate logits gamma [H]
    (float32). The routing seeds and fixed queries are the workload's Qseed and Qf."""
    X: np.ndarray
    Wk: np.ndarray
    Wv: np.ndarray
    Ws: np.ndarray
    Wo: np.ndarray
    bk: np.ndarray
    bv: np.ndarray
    bs: np.ndarray
    bo: np.ndarray
    nk: np.ndarray
    nq: np.ndarray
    gamma: np.ndarray
    dtype: str

    def f64(self, field: str) -> np.ndarray:
        if field == "gamma":
            return self.gamma.astype(np.float64)
        return to_float64(getattr(self, field), self.dtype)


def make_block_inputs(w: Workload, init: str = "random", seed: int | None = None) -> BlockInputs:
    """Seeded block inputs of the workload's shape and family.

    X: ``gauss`` draws N(0, 1); the mesh kinds draw fresh points of their family and embed the same
    11 features phi(x) with a pointwise input projection W_in in R^{11 x C} of N(0, 1/11) entries.
    ``init="identity"`` is the pages' initialization of the feature projections (W = I + Delta W,
    Delta W ~ N(0, 0.02^2) truncated at two standard deviations, zero biases, unit scales, gate logits
    0.25); the output projection gets the same form. ``init="random"`` draws dense N(0, 1/C) matrices,
    N(0, 0.1^2) biases, scales 1 + N(0, 0.2^2) and gate logits N(0.25, 1), so that no projection is
    close to a symmetric one.
    """
    C = w.H * w.D
    rng = np.random.Generator(np.random.PCG64(workload_seed(0) + 15485863 if seed is None else seed))
    kind = w.kind
    if kind == "gauss":
        X = rng.standard_normal((w.B, w.N, C))
    else:
        freqs = rng.normal(0.0, 2.0, size=(8, 3))
        w_in = rng.standard_normal((11, C)) / math.sqrt(11.0)
        X = np.empty((w.B, w.N, C))
        for b in range(w.B):
            pts = rng.random((w.N, 3)) if kind == "cube" else _sphere_surface_points(rng, w.N)
            X[b] = np.concatenate([pts, np.sin(pts @ freqs.T)], axis=1) @ w_in
    if init == "identity":
        def mat():
            d = rng.standard_normal((C, C)) * 0.02
            return np.eye(C) + np.clip(d, -0.04, 0.04)
        Ws = [mat() for _ in range(4)]
        bias = [np.zeros(C) for _ in range(4)]
        nk, nq = np.ones(w.D), np.ones(w.D)
        gamma = np.full(w.H, 0.25)
    elif init == "random":
        Ws = [rng.standard_normal((C, C)) / math.sqrt(C) for _ in range(4)]
        bias = [rng.standard_normal(C) * 0.1 for _ in range(4)]
        nk, nq = 1.0 + 0.2 * rng.standard_normal(w.D), 1.0 + 0.2 * rng.standard_normal(w.D)
        gamma = 0.25 + rng.standard_normal(w.H)
    else:
        raise ValueError(f"unknown init {init!r}")
    st = lambda a: _store(a, w.dtype)
    return BlockInputs(st(X), *(st(m) for m in Ws), *(st(b) for b in bias), st(nk), st(nq),
                       gamma.astype(np.float32), w.dtype)
