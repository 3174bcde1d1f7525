"""Python binding of the FLARE++ mixer library (libflarepp.so, C ABI in include/flarepp.h).

Argument marshalling only: torch tensors supply device memory and the stream; every step of the
mixer runs in the library's HIP kernels. The functions carry the C entry points' names. There is
no CPU fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# FLAREPP_LIB may name another build of the same library (for side-by-side timing).
LIB_PATH = os.environ.get("FLAREPP_LIB") or os.path.join(PKG_DIR, "libflarepp.so")

FLAREPP_OK = 0
FLAREPP_INVALID_ARGUMENT = 1
FLAREPP_UNSUPPORTED = 2
FLAREPP_MISALIGNED = 3
FLAREPP_OUT_OF_MEMORY = 4
FLAREPP_LAUNCH_FAILED = 5
FLAREPP_DEVICE_ERROR = 6
FLAREPP_SCRATCH_TOO_SMALL = 7
# Bytes of the static device scratch of flarepp_mix_noalloc (FLAREPP_NOALLOC_SCRATCH_BYTES).
FLAREPP_NOALLOC_SCRATCH_BYTES = 32 << 20
FLAREPP_FP32 = 0
FLAREPP_BF16 = 1

_lib = None


class FlareppError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {flarepp_strerror(status)} (status {status})" if what else
                         f"{flarepp_strerror(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library with its C signatures declared. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_latent_routing_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    mix_args = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, vp]
    L.flarepp_mix.argtypes = mix_args + [vp]
    L.flarepp_mix.restype = i32
    L.flarepp_mix_noalloc.argtypes = mix_args + [vp]
    L.flarepp_mix_noalloc.restype = i32
    L.flarepp_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.flarepp_workspace_bytes.restype = sz
    L.flarepp_mix_ws.argtypes = mix_args + [vp, sz, vp]
    L.flarepp_mix_ws.restype = i32
    L.flarepp_mix_debug.argtypes = mix_args + [vp, vp, vp, vp, sz, vp]
    L.flarepp_mix_debug.restype = i32
    flare_args = [vp, vp, vp, i32, i32, i64, i32, i32, i32, vp]
    L.flarepp_flare.argtypes = flare_args + [vp]
    L.flarepp_flare.restype = i32
    L.flarepp_flare_ws.argtypes = flare_args + [vp, sz, vp]
    L.flarepp_flare_ws.restype = i32
    simp_args = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, vp]
    L.flarepp_mix_simplified.argtypes = simp_args + [vp]
    L.flarepp_mix_simplified.restype = i32
    L.flarepp_mix_simplified_ws.argtypes = simp_args + [vp, sz, vp]
    L.flarepp_mix_simplified_ws.restype = i32
    bwd_args = mix_args[:6] + [vp, i32, i32, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.flarepp_mix_backward.argtypes = bwd_args + [vp]
    L.flarepp_mix_backward.restype = i32
    L.flarepp_mix_backward_ws.argtypes = bwd_args + [vp, sz, vp]
    L.flarepp_mix_backward_ws.restype = i32
    L.flarepp_mix_forward_saved.argtypes = mix_args + [vp, sz, vp]
    L.flarepp_mix_forward_saved.restype = i32
    L.flarepp_mix_backward_saved.argtypes = bwd_args + [vp, sz, vp]
    L.flarepp_mix_backward_saved.restype = i32
    L.flarepp_backward_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.flarepp_backward_workspace_bytes.restype = sz
    L.flarepp_project.argtypes = [vp] * 8 + [i32, i32, i64, i32, i32, vp, vp, vp, vp]
    L.flarepp_project.restype = i32
    L.flarepp_out_project.argtypes = [vp, vp, vp, i32, i32, i64, i32, i32, vp, vp]
    L.flarepp_out_project.restype = i32
    L.flarepp_block_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.flarepp_block_workspace_bytes.restype = sz
    block_args = [vp] * 14 + [i32, i32, i64, i32, i32, i32, vp]
    L.flarepp_block.argtypes = block_args + [vp]
    L.flarepp_block.restype = i32
    L.flarepp_block_ws.argtypes = block_args + [vp, sz, vp]
    L.flarepp_block_ws.restype = i32
    L.flarepp_debug_force_exact.argtypes = [i32]
    L.flarepp_debug_force_exact.restype = i32
    L.flarepp_timing_enable.argtypes = [i32]
    L.flarepp_timing_enable.restype = i32
    L.flarepp_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong), i32]
    L.flarepp_timing_read.restype = i32
    L.flarepp_kernel_name.argtypes = [i32]
    L.flarepp_kernel_name.restype = ctypes.c_char_p
    L.flarepp_strerror.argtypes = [i32]
    L.flarepp_strerror.restype = ctypes.c_char_p
    L.flarepp_version.argtypes = []
    L.flarepp_version.restype = i32
    _lib = L
    return L


def flarepp_strerror(status: int) -> str:
    return lib().flarepp_strerror(int(status)).decode()


def flarepp_version() -> int:
    return int(lib().flarepp_version())


def flarepp_kernel_name(i: int):
    r = lib().flarepp_kernel_name(int(i))
    return None if r is None else r.decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FLAREPP_FP32
    if t.dtype == torch.bfloat16:
        return FLAREPP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _shapes(K, V, S, Qseed, Qf, g):
    import torch
    if K.dim() != 4:
        raise ValueError("K, V, S must be [B, H, N, D]")
    B, H, N, D = K.shape
    if V.shape != K.shape or S.shape != K.shape:
        raise ValueError("K, V, S must have the same shape")
    if Qseed.dim() != 3 or Qseed.shape[0] != H or Qseed.shape[2] != D or Qf.shape != Qseed.shape:
        raise ValueError("Qseed and Qf must be [H, M, D]")
    if g.shape != (H,) or g.dtype != torch.float32:
        raise ValueError("g must be a float32 tensor of shape [H]")
    for t in (K, V, S, Qseed, Qf, g):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    for t in (V, S, Qseed, Qf):
        if t.dtype != K.dtype:
            raise ValueError("K, V, S, Qseed, Qf must share one dtype")
    return B, H, N, Qseed.shape[1], D


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _check(status: int, what: str):
    if status != FLAREPP_OK:
        raise FlareppError(status, what)


def _require_like(name, t, shape, dtype):
    """A caller-supplied output: a contiguous tensor of the given shape and dtype."""
    import torch
    if not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def _require_device(ref, **tensors):
    """Every tensor (None entries skipped) lives on ref's GPU: the kernels read and write them
    there, so a host tensor or another GPU's memory would be a fault, not an error."""
    import torch
    if not isinstance(ref, torch.Tensor) or ref.device.type != "cuda":
        raise ValueError("the mixer's tensors must be on a GPU (device 'cuda')")
    for name, t in tensors.items():
        if t is not None and (not isinstance(t, torch.Tensor) or t.device != ref.device):
            raise ValueError(f"{name} must be on {ref.device}, the device of the other tensors")


def _require_workspace(workspace, device):
    """A caller-owned workspace: a contiguous uint8 tensor on the mixer's GPU (its numel() is the
    byte count the library checks against the size it needs)."""
    import torch
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}")


def flarepp_workspace_bytes(B: int, H: int, N: int, M: int, D: int, dtype: int) -> int:
    return int(lib().flarepp_workspace_bytes(B, H, N, M, D, dtype))


def flarepp_mix(K, V, S, Qseed, Qf, g, out=None, stream=None):
    """FLARE++ mixer forward. K, V, S: [B, H, N, D]; Qseed, Qf: [H, M, D] (float32 or bfloat16,
    one dtype, on one GPU); g: [H] float32 gate values. Returns out [B, H, N, D]. The library
    allocates its workspace stream-ordered."""
    import torch
    B, H, N, M, D = _shapes(K, V, S, Qseed, Qf, g)
    if out is not None:
        _require_like("out", out, K.shape, K.dtype)
    _require_device(K, V=V, S=S, Qseed=Qseed, Qf=Qf, g=g, out=out)
    if out is None:
        out = torch.empty_like(K)
    st = lib().flarepp_mix(_ptr(K), _ptr(V), _ptr(S), _ptr(Qseed), _ptr(Qf), _ptr(g), B, H, N, M, D,
                           _dtype_code(K), _ptr(out), _stream_ptr(stream, K.device))
    _check(st, "flarepp_mix")
    return out


def flarepp_mix_noalloc(K, V, S, Qseed, Qf, g, out=None, stream=None):
    """flarepp_mix with its workspace in the library's static device scratch: the C call allocates
    nothing (for callers that cannot allocate). Calls that overlap on one GPU race; problems whose
    workspace exceeds FLAREPP_NOALLOC_SCRATCH_BYTES raise (status FLAREPP_SCRATCH_TOO_SMALL). `out`
    should be supplied by a caller that cannot allocate (torch allocates it otherwise)."""
    import torch
    B, H, N, M, D = _shapes(K, V, S, Qseed, Qf, g)
    if out is not None:
        _require_like("out", out, K.shape, K.dtype)
    _require_device(K, V=V, S=S, Qseed=Qseed, Qf=Qf, g=g, out=out)
    if out is None:
        out = torch.empty_like(K)
    st = lib().flarepp_mix_noalloc(_ptr(K), _ptr(V), _ptr(S), _ptr(Qseed), _ptr(Qf), _ptr(g), B, H, N, M, D,
                                   _dtype_code(K), _ptr(out), _stream_ptr(stream, K.device))
    _check(st, "flarepp_mix_noalloc")
    return out


def _workspace(B, H, N, M, D, dt, device, workspace):
    import torch
    need = flarepp_workspace_bytes(B, H, N, M, D, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    else:
        _require_workspace(workspace, device)
    return workspace, need


def flarepp_mix_ws(K, V, S, Qseed, Qf, g, out=None, workspace=None, stream=None):
    """flarepp_mix with a torch-owned workspace (a uint8 tensor of flarepp_workspace_bytes bytes;
    allocated here when not given)."""
    import torch
    B, H, N, M, D = _shapes(K, V, S, Qseed, Qf, g)
    dt = _dtype_code(K)
    if out is not None:
        _require_like("out", out, K.shape, K.dtype)
    _require_device(K, V=V, S=S, Qseed=Qseed, Qf=Qf, g=g, out=out)
    if out is None:
        out = torch.empty_like(K)
    workspace, _ = _workspace(B, H, N, M, D, dt, K.device, workspace)
    st = lib().flarepp_mix_ws(_ptr(K), _ptr(V), _ptr(S), _ptr(Qseed), _ptr(Qf), _ptr(g), B, H, N, M, D, dt,
                              _ptr(out), _ptr(workspace), workspace.numel(), _stream_ptr(stream, K.device))
    _check(st, "flarepp_mix_ws")
    return out


def flarepp_mix_debug(K, V, S, Qseed, Qf, g, out=None, workspace=None, stream=None):
    """flarepp_mix_ws that also returns the fp32 latent stages Qd, Q, Z, each [B, H, M, D]."""
    import torch
    B, H, N, M, D = _shapes(K, V, S, Qseed, Qf, g)
    dt = _dtype_code(K)
    if out is not None:
        _require_like("out", out, K.shape, K.dtype)
    _require_device(K, V=V, S=S, Qseed=Qseed, Qf=Qf, g=g, out=out)
    if out is None:
        out = torch.empty_like(K)
    workspace, _ = _workspace(B, H, N, M, D, dt, K.device, workspace)
    Qd, Q, Z = (torch.empty((B, H, M, D), dtype=torch.float32, device=K.device) for _ in range(3))
    st = lib().flarepp_mix_debug(_ptr(K), _ptr(V), _ptr(S), _ptr(Qseed), _ptr(Qf), _ptr(g), B, H, N, M, D, dt,
                                 _ptr(out), _ptr(Qd), _ptr(Q), _ptr(Z), _ptr(workspace), workspace.numel(),
                                 _stream_ptr(stream, K.device))
    _check(st, "flarepp_mix_debug")
    return out, Qd, Q, Z


def _flare_shapes(K, V, Q):
    if K.dim() != 4 or V.shape != K.shape:
        raise ValueError("K and V must be [B, H, N, D] of one shape")
    B, H, N, D = K.shape
    if Q.dim() != 3 or Q.shape[0] != H or Q.shape[2] != D:
        raise ValueError("Q must be [H, M, D]")
    for t in (K, V, Q):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if t.dtype != K.dtype:
            raise ValueError("K, V, Q must share one dtype")
    return B, H, N, Q.shape[1], D


def flarepp_flare(K, V, Q, out=None, workspace=None, stream=None):
    """Plain FLARE (Eq. 3): out = softmax_M(K Q^T/sqrt(D)) softmax_N(Q K^T/sqrt(D)) V with the
    fixed latent queries Q [H, M, D] used as given. With `workspace` (a uint8 tensor of
    flarepp_workspace_bytes bytes) the caller owns the workspace (flarepp_flare_ws)."""
    import torch
    B, H, N, M, D = _flare_shapes(K, V, Q)
    dt = _dtype_code(K)
    if out is not None:
        _require_like("out", out, K.shape, K.dtype)
    _require_device(K, V=V, Q=Q, out=out)
    if workspace is not None:
        _require_workspace(workspace, K.device)
    if out is None:
        out = torch.empty_like(K)
    if workspace is None:
        st = lib().flarepp_flare(_ptr(K), _ptr(V), _ptr(Q), B, H, N, M, D, dt, _ptr(out), _stream_ptr(stream, K.device))
        _check(st, "flarepp_flare")
    else:
        st = lib().flarepp_flare_ws(_ptr(K), _ptr(V), _ptr(Q), B, H, N, M, D, dt, _ptr(out), _ptr(workspace),
                                    workspace.numel(), _stream_ptr(stream, K.device))
        _check(st, "flarepp_flare_ws")
    return out


def flarepp_backward_workspace_bytes(B: int, H: int, N: int, M: int, D: int, dtype: int) -> int:
    return int(lib().flarepp_backward_workspace_bytes(B, H, N, M, D, dtype))


def flarepp_mix_backward(K, V, S, Qseed, Qf, g, dY, grads=None, workspace=None, stream=None, _saved=False):
    """Backward pass of flarepp_mix given the output cotangent dY [B, H, N, D] (the input dtype).
    Returns {dK, dV, dS: [B, H, N, D], dQseed, dQf: [H, M, D] in the input dtype, dg: [H] float32};
    `grads` may supply those tensors. With `workspace` (a uint8 tensor of
    flarepp_backward_workspace_bytes bytes) the caller owns the workspace (flarepp_mix_backward_ws)."""
    import torch
    B, H, N, M, D = _shapes(K, V, S, Qseed, Qf, g)
    if dY.shape != K.shape or dY.dtype != K.dtype or not dY.is_contiguous():
        raise ValueError("dY must be a contiguous tensor of K's shape and dtype")
    dt = _dtype_code(K)
    if grads is not None:
        expect = {"dK": K, "dV": K, "dS": K, "dQseed": Qseed, "dQf": Qf, "dg": g}
        for name, like in expect.items():
            if name not in grads:
                raise ValueError(f"grads must hold {name}")
            _require_like(f"grads[{name!r}]", grads[name], like.shape, like.dtype)
    _require_device(K, V=V, S=S, Qseed=Qseed, Qf=Qf, g=g, dY=dY,
                    **({f"grads[{k!r}]": v for k, v in grads.items()} if grads is not None else {}))
    if workspace is not None:
        _require_workspace(workspace, K.device)
    if grads is None:
        grads = {"dK": torch.empty_like(K), "dV": torch.empty_like(K), "dS": torch.empty_like(K),
                 "dQseed": torch.empty_like(Qseed), "dQf": torch.empty_like(Qf), "dg": torch.empty_like(g)}
    outs = [_ptr(grads[k]) for k in ("dK", "dV", "dS", "dQseed", "dQf", "dg")]
    args = [_ptr(K), _ptr(V), _ptr(S), _ptr(Qseed), _ptr(Qf), _ptr(g), _ptr(dY), B, H, N, M, D, dt] + outs
    if _saved:
        if workspace is None:
            raise ValueError("flarepp_mix_backward_saved needs the workspace of flarepp_mix_forward_saved")
        st = lib().flarepp_mix_backward_saved(*args, _ptr(workspace), workspace.numel(), _stream_ptr(stream, K.device))
        _check(st, "flarepp_mix_backward_saved")
    elif workspace is None:
        st = lib().flarepp_mix_backward(*args, _stream_ptr(stream, K.device))
        _check(st, "flarepp_mix_backward")
    else:
        st = lib().flarepp_mix_backward_ws(*args, _ptr(workspace), workspace.numel(), _stream_ptr(stream, K.device))
        _check(st, "flarepp_mix_backward_ws")
    return grads


def flarepp_mix_forward_saved(K, V, S, Qseed, Qf, g, workspace, out=None, stream=None):
    """The mixer forward of a training step: writes out [B, H, N, D] and keeps in `workspace` (a uint8
    tensor of at least flarepp_backward_workspace_bytes bytes, kept by the caller) the state
    flarepp_mix_backward_saved starts from. Returns out."""
    import torch
    B, H, N, M, D = _shapes(K, V, S, Qseed, Qf, g)
    if out is not None:
        _require_like("out", out, K.shape, K.dtype)
    _require_device(K, V=V, S=S, Qseed=Qseed, Qf=Qf, g=g, out=out)
    _require_workspace(workspace, K.device)
    if out is None:
        out = torch.empty_like(K)
    st = lib().flarepp_mix_forward_saved(_ptr(K), _ptr(V), _ptr(S), _ptr(Qseed), _ptr(Qf), _ptr(g), B, H, N, M, D,
                                         _dtype_code(K), _ptr(out), _ptr(workspace), workspace.numel(),
                                         _stream_ptr(stream, K.device))
    _check(st, "flarepp_mix_forward_saved")
    return out


def flarepp_mix_backward_saved(K, V, S, Qseed, Qf, g, dY, workspace, grads=None, stream=None):
    """flarepp_mix_backward from the state flarepp_mix_forward_saved left in `workspace` for the same
    inputs (no recompute). Returns the cotangents as flarepp_mix_backward does."""
    return flarepp_mix_backward(K, V, S, Qseed, Qf, g, dY, grads=grads, workspace=workspace, stream=stream,
                                _saved=True)


def flarepp_mix_simplified(K, V, Sk, Sv, Qseed, out=None, workspace=None, stream=None):
    """Simplified FLARE++ (Eq. 20): routing queries Qd = SDPA(Qseed, Sk, Sv) alone, then encode and
    decode. K, V, Sk, Sv: [B, H, N, D]; Qseed: [H, M, D] (one dtype). With `workspace` (a uint8 tensor
    of flarepp_workspace_bytes bytes) the caller owns the workspace (flarepp_mix_simplified_ws)."""
    import torch
    if K.dim() != 4 or any(t.shape != K.shape for t in (V, Sk, Sv)):
        raise ValueError("K, V, Sk, Sv must be [B, H, N, D] of one shape")
    B, H, N, D = K.shape
    if Qseed.dim() != 3 or Qseed.shape[0] != H or Qseed.shape[2] != D:
        raise ValueError("Qseed must be [H, M, D]")
    for t in (K, V, Sk, Sv, Qseed):
        if not t.is_contiguous() or t.dtype != K.dtype:
            raise ValueError("all tensors must be contiguous and share one dtype")
    M = Qseed.shape[1]
    dt = _dtype_code(K)
    if out is not None:
        _require_like("out", out, K.shape, K.dtype)
    _require_device(K, V=V, Sk=Sk, Sv=Sv, Qseed=Qseed, out=out)
    if workspace is not None:
        _require_workspace(workspace, K.device)
    if out is None:
        out = torch.empty_like(K)
    args = [_ptr(K), _ptr(V), _ptr(Sk), _ptr(Sv), _ptr(Qseed), B, H, N, M, D, dt, _ptr(out)]
    if workspace is None:
        st = lib().flarepp_mix_simplified(*args, _stream_ptr(stream, K.device))
        _check(st, "flarepp_mix_simplified")
    else:
        st = lib().flarepp_mix_simplified_ws(*args, _ptr(workspace), workspace.numel(), _stream_ptr(stream, K.device))
        _check(st, "flarepp_mix_simplified_ws")
    return out


def _linear_args(X, weights, biases, scales, H):
    """Checks of the projections' arguments: X [B, N, C] (C = H D), weights [C, C] in torch Linear's
    [out, in] layout, biases [C] and scales [D] optional, one dtype, contiguous."""
    if X.dim() != 3 or X.shape[-1] % H:
        raise ValueError("X must be [B, N, C] with C divisible by H")
    C = X.shape[-1]
    D = C // H
    for W in weights:
        if W.shape != (C, C):
            raise ValueError("projection weights must be [C, C]")
    for b in biases:
        if b is not None and b.shape != (C,):
            raise ValueError("biases must be [C]")
    for sc in scales:
        if sc is not None and sc.shape != (D,):
            raise ValueError("normalization scales must be [D]")
    for t in (X, *weights, *biases, *scales):
        if t is not None and (not t.is_contiguous() or t.dtype != X.dtype):
            raise ValueError("all tensors must be contiguous and share X's dtype")
    return X.shape[0], X.shape[1], C, D


def flarepp_project(X, Wk, Wv, Ws, H, bk=None, bv=None, bs=None, nk=None, out=None, stream=None):
    """The projections in front of the mixer: K = N_a(X Wk^T + bk) (scale nk), V = X Wv^T + bv and
    S = X Ws^T + bs, each [B, H, N, D]. X: [B, N, C]; W*: [C, C] (torch Linear layout); biases [C] and
    nk [D] optional. Returns (K, V, S); `out` may supply them."""
    import torch
    B, N, C, D = _linear_args(X, (Wk, Wv, Ws), (bk, bv, bs), (nk,), H)
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be a tuple (K, V, S)")
        for name, t in zip("KVS", out):
            _require_like(f"out {name}", t, (B, H, N, D), X.dtype)
    _require_device(X, Wk=Wk, Wv=Wv, Ws=Ws, bk=bk, bv=bv, bs=bs, nk=nk,
                    **({f"out {n}": t for n, t in zip("KVS", out)} if out is not None else {}))
    if out is None:
        out = tuple(torch.empty((B, H, N, D), dtype=X.dtype, device=X.device) for _ in range(3))
    K, V, S = out
    st = lib().flarepp_project(_ptr(X), _ptr(Wk), _ptr(Wv), _ptr(Ws), _ptr(bk), _ptr(bv), _ptr(bs), _ptr(nk),
                               B, H, N, D, _dtype_code(X), _ptr(K), _ptr(V), _ptr(S), _stream_ptr(stream, X.device))
    _check(st, "flarepp_project")
    return K, V, S


def flarepp_out_project(Y, Wo, bo=None, out=None, stream=None):
    """The output projection: out[b, n] = concat_h(Y[b, h, n]) Wo^T + bo for Y [B, H, N, D]; Wo [C, C]
    (torch Linear layout), bo [C] optional. Returns out [B, N, C]."""
    import torch
    if Y.dim() != 4:
        raise ValueError("Y must be [B, H, N, D]")
    B, H, N, D = Y.shape
    C = H * D
    if Wo.shape != (C, C) or (bo is not None and bo.shape != (C,)):
        raise ValueError("Wo must be [C, C] and bo [C]")
    for t in (Y, Wo, bo):
        if t is not None and (not t.is_contiguous() or t.dtype != Y.dtype):
            raise ValueError("all tensors must be contiguous and share Y's dtype")
    if out is not None:
        _require_like("out", out, (B, N, C), Y.dtype)
    _require_device(Y, Wo=Wo, bo=bo, out=out)
    if out is None:
        out = torch.empty((B, N, C), dtype=Y.dtype, device=Y.device)
    st = lib().flarepp_out_project(_ptr(Y), _ptr(Wo), _ptr(bo), B, H, N, D, _dtype_code(Y), _ptr(out),
                                   _stream_ptr(stream, Y.device))
    _check(st, "flarepp_out_project")
    return out


def flarepp_block_workspace_bytes(B: int, H: int, N: int, M: int, D: int, dtype: int) -> int:
    return int(lib().flarepp_block_workspace_bytes(B, H, N, M, D, dtype))


def flarepp_block(X, Wk, Wv, Ws, Wo, Qseed, Qf, gamma, bk=None, bv=None, bs=None, bo=None, nq=None, nk=None,
                  out=None, workspace=None, stream=None):
    """The mixer block: projections, the mixer with seeds N_a(Qseed) (scale nq) and gates
    sigmoid(gamma), and the output projection. X: [B, N, C]; W*: [C, C] (torch Linear layout);
    Qseed, Qf: [H, M, D]; gamma: [H] float32; biases [C], nq and nk [D] optional. Returns out
    [B, N, C]. With `workspace` (a uint8 tensor of flarepp_block_workspace_bytes bytes) the caller
    owns the workspace (flarepp_block_ws)."""
    import torch
    if Qseed.dim() != 3 or Qf.shape != Qseed.shape:
        raise ValueError("Qseed and Qf must be [H, M, D]")
    H, M, D = Qseed.shape
    B, N, C, D2 = _linear_args(X, (Wk, Wv, Ws, Wo), (bk, bv, bs, bo), (nq, nk), H)
    if D2 != D:
        raise ValueError("X's channels must be H * D")
    for t in (Qseed, Qf):
        if not t.is_contiguous() or t.dtype != X.dtype:
            raise ValueError("Qseed and Qf must be contiguous and share X's dtype")
    if gamma.shape != (H,) or gamma.dtype != torch.float32 or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous float32 tensor of shape [H]")
    if out is not None:
        _require_like("out", out, (B, N, C), X.dtype)
    _require_device(X, Wk=Wk, Wv=Wv, Ws=Ws, Wo=Wo, bk=bk, bv=bv, bs=bs, bo=bo, Qseed=Qseed, Qf=Qf, gamma=gamma,
                    nq=nq, nk=nk, out=out)
    if workspace is not None:
        _require_workspace(workspace, X.device)
    if out is None:
        out = torch.empty((B, N, C), dtype=X.dtype, device=X.device)
    args = [_ptr(t) for t in (X, Wk, Wv, Ws, Wo, bk, bv, bs, bo, Qseed, Qf, gamma, nq, nk)]
    args += [B, H, N, M, D, _dtype_code(X), _ptr(out)]
    if workspace is None:
        st = lib().flarepp_block(*args, _stream_ptr(stream, X.device))
        _check(st, "flarepp_block")
    else:
        st = lib().flarepp_block_ws(*args, _ptr(workspace), workspace.numel(), _stream_ptr(stream, X.device))
        _check(st, "flarepp_block_ws")
    return out


def flarepp_debug_force_exact(enable: bool = True) -> bool:
    """Test hook: force the exact (running-maximum) softmax path for all later calls in this
    process. Returns the previous setting."""
    return bool(lib().flarepp_debug_force_exact(1 if enable else 0))


def flarepp_timing_enable(enable: bool = True) -> None:
    lib().flarepp_timing_enable(1 if enable else 0)


def flarepp_timing_read() -> dict:
    """Per-kernel event timings accumulated since the last read: {name: (total_ms, launches)}."""
    n = 32
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_longlong * n)()
    k = lib().flarepp_timing_read(ms, cnt, n)
    if k < 0:
        raise FlareppError(-k, "flarepp_timing_read")
    return {flarepp_kernel_name(i): (ms[i], cnt[i]) for i in range(k)}


__all__ = ["FlareppError", "flarepp_mix", "flarepp_mix_ws", "flarepp_mix_noalloc", "FLAREPP_NOALLOC_SCRATCH_BYTES", "flarepp_mix_debug", "flarepp_workspace_bytes",
           "flarepp_flare", "flarepp_mix_simplified", "flarepp_mix_backward", "flarepp_backward_workspace_bytes",
           "flarepp_mix_forward_saved", "flarepp_mix_backward_saved",
           "flarepp_project", "flarepp_out_project", "flarepp_block", "flarepp_block_workspace_bytes",
           "flarepp_debug_force_exact", "flarepp_timing_enable", "flarepp_timing_read", "flarepp_kernel_name", "flarepp_strerror",
           "flarepp_version", "lib", "FLAREPP_FP32", "FLAREPP_BF16"]
