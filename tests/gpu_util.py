"""Helpers shared by the GPU parity tests: device copies of a workload, a call through the C ABI,
the oracle's results for the same inputs, and the parity metrics."""
from __future__ import annotations

import sys

import numpy as np

import oracle

#: fp32 bar: max |Y - Y_ref| / max |Y_ref| per (b, h) slice.
TOL_FP32 = 1e-5
#: bf16 bar: max |Y - Y_ref| / RMS(Y_ref) per (b, h) slice (bf16 inputs, fp32 accumulation).
TOL_BF16 = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_device(w):
    import torch

    def t(arr):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()

    return dict(K=t(w.K), V=t(w.V), S=t(w.S), Qseed=t(w.Qseed), Qf=t(w.Qf),
                g=__import__("torch").from_numpy(np.ascontiguousarray(w.g)).cuda())


def run_gpu(w, debug=True, dev=None):
    """One mixer call on the GPU. Returns float64 numpy Y [B,H,N,D] and (if debug) Qd, Q, Z."""
    import torch
    from rank_latent_routing_amd import flarepp_mix_debug, flarepp_mix_ws
    dev = dev or to_device(w)
    args = (dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"])
    if debug:
        out, Qd, Q, Z = flarepp_mix_debug(*args)
        torch.cuda.synchronize()
        return (out.float().cpu().numpy().astype(np.float64), Qd.cpu().numpy().astype(np.float64),
                Q.cpu().numpy().astype(np.float64), Z.cpu().numpy().astype(np.float64))
    out = flarepp_mix_ws(*args)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def oracle_head(w, b, h, block=None):
    """The oracle's stages for slice (b, h) of a workload (Qd, Q, Z, Y in float64)."""
    from workloads import to_float64
    K = to_float64(w.K[b, h], w.dtype)
    V = to_float64(w.V[b, h], w.dtype)
    S = to_float64(w.S[b, h], w.dtype)
    Qs = to_float64(w.Qseed[h], w.dtype)
    Qf = to_float64(w.Qf[h], w.dtype)
    return oracle.mix_head(K, V, S, Qs, Qf, float(w.g[h]), block=block)


def slice_err(got, ref, dtype):
    """Parity metric of one (b, h) slice."""
    d = np.abs(got - ref).max()
    if dtype == "fp32":
        return d / max(np.abs(ref).max(), 1e-30)
    return d / max(np.sqrt(np.mean(ref * ref)), 1e-30)


def tol(dtype):
    return TOL_FP32 if dtype == "fp32" else TOL_BF16
