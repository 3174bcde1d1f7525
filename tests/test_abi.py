"""Host-side checks of the C ABI: the library loads, exports every entry point the header declares,
and rejects bad arguments before it touches a GPU. No kernel is launched here."""
import ctypes
import os
import re

import pytest

import rank_latent_routing_amd as fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flarepp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flarepp_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return fl.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(L):
    assert fl.flarepp_version() >= 100
    for s in range(0, 8):
        assert isinstance(fl.flarepp_strerror(s), str) and fl.flarepp_strerror(s)
    assert [fl.flarepp_kernel_name(i) for i in range(6)] == [
        "synthesis_partial", "merge_gate", "encode_partial", "merge", "decode", "query_prep"]
    assert [fl.flarepp_kernel_name(i) for i in range(6, 16)] == [
        "bwd_center", "bwd_token_decode", "bwd_latent_decode", "bwd_reduce_decode", "bwd_latent_encode",
        "bwd_reduce_gate", "bwd_latent_synthesis", "bwd_reduce_synthesis", "bwd_token_encode",
        "bwd_token_synthesis"]
    assert [fl.flarepp_kernel_name(i) for i in range(16, 19)] == ["project", "out_project", "block_params"]
    assert fl.flarepp_kernel_name(19) is None


def _mix(L, K=0x1000, V=0x2000, S=0x3000, Qs=0x4000, Qf=0x5000, g=0x6000, B=1, H=1, N=64, M=8, D=16,
         dtype=1, out=0x7000000):
    vp = ctypes.c_void_p
    return L.flarepp_mix(vp(K), vp(V), vp(S), vp(Qs), vp(Qf), vp(g), B, H, N, M, D, dtype, vp(out), vp(0))


def test_size_validation(L):
    assert _mix(L, D=24) == fl.FLAREPP_UNSUPPORTED
    assert _mix(L, D=64) == fl.FLAREPP_UNSUPPORTED
    assert _mix(L, M=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _mix(L, M=513) == fl.FLAREPP_UNSUPPORTED
    assert _mix(L, dtype=7) == fl.FLAREPP_UNSUPPORTED
    assert _mix(L, N=-1) == fl.FLAREPP_INVALID_ARGUMENT
    assert _mix(L, B=-2) == fl.FLAREPP_INVALID_ARGUMENT
    assert _mix(L, B=300, H=300) == fl.FLAREPP_UNSUPPORTED


def test_pointer_validation(L):
    assert _mix(L, K=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _mix(L, g=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _mix(L, out=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _mix(L, V=0x2008) == fl.FLAREPP_MISALIGNED
    assert _mix(L, out=0x7000004) == fl.FLAREPP_MISALIGNED
    # out overlapping an input
    assert _mix(L, out=0x1000 + 64) == fl.FLAREPP_INVALID_ARGUMENT


def test_empty_problem_is_a_no_op(L):
    # B*H*N == 0: nothing to compute, nothing enqueued, no device needed.
    assert _mix(L, N=0) == fl.FLAREPP_OK
    assert _mix(L, B=0, K=0, V=0, S=0) == fl.FLAREPP_OK
    assert fl.flarepp_workspace_bytes(1, 1, 0, 8, 16, 1) == 0


def test_workspace_bytes(L):
    # Invalid sizes give 0; valid ones hold the chunk partials and the two latent tensors.
    assert fl.flarepp_workspace_bytes(1, 1, 100, 0, 16, 1) == 0
    assert fl.flarepp_workspace_bytes(1, 1, 100, 8, 24, 1) == 0
    for (B, H, N, M, D, dt) in [(1, 2, 1024, 32, 16, 0), (4, 8, 16384, 64, 16, 1), (32, 8, 4096, 128, 32, 1),
                                (2, 8, 65536, 256, 32, 1), (1, 8, 1 << 20, 512, 32, 1), (3, 5, 1, 1, 32, 0)]:
        ws = fl.flarepp_workspace_bytes(B, H, N, M, D, dt)
        es = 2 if dt == 1 else 4
        m32 = (M + 31) // 32 * 32
        m16 = (M + 15) // 16 * 16
        assert ws % 256 == 0
        assert ws >= 2 * B * H * m32 * D * es + B * H * m16 * (D + 2) * 4
        assert ws < 64 * 2 ** 20 + 2 * B * H * m32 * D * es  # partials stay small against the inputs


def test_workspace_too_small_is_rejected(L):
    vp = ctypes.c_void_p
    need = fl.flarepp_workspace_bytes(1, 1, 64, 8, 16, 1)
    rc = L.flarepp_mix_ws(vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), vp(0x5000), vp(0x6000), 1, 1, 64, 8,
                          16, 1, vp(0x7000000), vp(0x9000000), need - 1, vp(0))
    assert rc == fl.FLAREPP_INVALID_ARGUMENT
    rc = L.flarepp_mix_ws(vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), vp(0x5000), vp(0x6000), 1, 1, 64, 8,
                          16, 1, vp(0x7000000), vp(0x9000010), need, vp(0))
    assert rc == fl.FLAREPP_MISALIGNED


def test_timing_read_without_records(L):
    fl.flarepp_timing_enable(False)
    t = fl.flarepp_timing_read()
    assert set(t) == {fl.flarepp_kernel_name(i) for i in range(19)}
    assert all(v == (0.0, 0) for v in t.values())


def _flare(L, K=0x1000, V=0x2000, Q=0x4000, B=1, H=1, N=64, M=8, D=16, dtype=1, out=0x7000000):
    vp = ctypes.c_void_p
    return L.flarepp_flare(vp(K), vp(V), vp(Q), B, H, N, M, D, dtype, vp(out), vp(0))


def test_flare_validation(L):
    assert _flare(L, D=24) == fl.FLAREPP_UNSUPPORTED
    assert _flare(L, M=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _flare(L, M=513) == fl.FLAREPP_UNSUPPORTED
    assert _flare(L, Q=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _flare(L, Q=0x4004) == fl.FLAREPP_MISALIGNED
    assert _flare(L, out=0x1000 + 64) == fl.FLAREPP_INVALID_ARGUMENT
    assert _flare(L, N=0) == fl.FLAREPP_OK
    vp = ctypes.c_void_p
    need = fl.flarepp_workspace_bytes(1, 1, 64, 8, 16, 1)
    rc = L.flarepp_flare_ws(vp(0x1000), vp(0x2000), vp(0x4000), 1, 1, 64, 8, 16, 1, vp(0x7000000), vp(0x9000000),
                            need - 1, vp(0))
    assert rc == fl.FLAREPP_INVALID_ARGUMENT


def _bwd(L, K=0x1000, V=0x2000, S=0x3000, Qs=0x4000, Qf=0x5000, g=0x6000, dY=0x8000000, B=1, H=1, N=64, M=8,
         D=16, dtype=1, dK=0x9000000, dV=0xA000000, dS=0xB000000, dQs=0xC000000, dQf=0xD000000, dg=0xE000000,
         ws=None, ws_bytes=0):
    vp = ctypes.c_void_p
    args = [vp(K), vp(V), vp(S), vp(Qs), vp(Qf), vp(g), vp(dY), B, H, N, M, D, dtype, vp(dK), vp(dV), vp(dS),
            vp(dQs), vp(dQf), vp(dg)]
    if ws is None:
        return L.flarepp_mix_backward(*args, vp(0))
    return L.flarepp_mix_backward_ws(*args, vp(ws), ws_bytes, vp(0))


def test_backward_validation(L):
    assert _bwd(L, D=24) == fl.FLAREPP_UNSUPPORTED
    assert _bwd(L, M=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _bwd(L, M=513) == fl.FLAREPP_UNSUPPORTED
    assert _bwd(L, dY=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _bwd(L, dg=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _bwd(L, dQs=0xC000004) == fl.FLAREPP_MISALIGNED
    # Outputs must not overlap inputs or each other.
    assert _bwd(L, dK=0x1000 + 64) == fl.FLAREPP_INVALID_ARGUMENT
    assert _bwd(L, dV=0x9000000 + 32) == fl.FLAREPP_INVALID_ARGUMENT
    assert _bwd(L, dg=0xD000000) == fl.FLAREPP_INVALID_ARGUMENT
    need = fl.flarepp_backward_workspace_bytes(1, 1, 64, 8, 16, 1)
    assert _bwd(L, ws=0xF0000000, ws_bytes=need - 1) == fl.FLAREPP_INVALID_ARGUMENT
    assert _bwd(L, ws=0xF0000010, ws_bytes=need) == fl.FLAREPP_MISALIGNED


def test_backward_workspace_bytes(L):
    assert fl.flarepp_backward_workspace_bytes(1, 1, 100, 0, 16, 1) == 0
    assert fl.flarepp_backward_workspace_bytes(1, 1, 0, 8, 16, 1) == 0
    assert fl.flarepp_backward_workspace_bytes(1, 1, 100, 513, 32, 0) == 0
    assert fl.flarepp_backward_workspace_bytes(1, 1, 100, 512, 32, 0) > 0
    for (B, H, N, M, D, dt) in [(1, 2, 1024, 32, 16, 0), (4, 8, 16384, 64, 16, 1), (1, 8, 1 << 20, 512, 32, 1)]:
        ws = fl.flarepp_backward_workspace_bytes(B, H, N, M, D, dt)
        es = 2 if dt == 1 else 4
        assert ws % 256 == 0
        # At least the forward's workspace and two per-token statistics, and for bf16 the decode
        # call's part of dK in fp32; nothing else token-sized.
        extra = B * H * N * (8 + (4 * D if dt == 1 else 0))
        assert ws >= fl.flarepp_workspace_bytes(B, H, N, M, D, dt) + extra
        assert ws < extra + 512 * 2 ** 20


def test_simplified_validation(L):
    vp = ctypes.c_void_p
    def call(K=0x1000, V=0x2000, Sk=0x3000, Sv=0x4000, Qs=0x5000, N=64, M=8, D=16, dtype=1, out=0x7000000):
        return L.flarepp_mix_simplified(vp(K), vp(V), vp(Sk), vp(Sv), vp(Qs), 1, 1, N, M, D, dtype, vp(out), vp(0))
    assert call(D=24) == fl.FLAREPP_UNSUPPORTED
    assert call(M=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(Sv=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(Sk=0x3008) == fl.FLAREPP_MISALIGNED
    assert call(out=0x4000 + 64) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(N=0) == fl.FLAREPP_OK


def _proj(L, X=0x1000, Wk=0x2000, Wv=0x3000, Ws=0x4000, bk=0, bv=0, bs=0, nk=0, B=1, H=2, N=64, D=16, dtype=1,
          K=0x7000000, V=0x8000000, S=0x9000000):
    vp = ctypes.c_void_p
    return L.flarepp_project(vp(X), vp(Wk), vp(Wv), vp(Ws), vp(bk), vp(bv), vp(bs), vp(nk), B, H, N, D, dtype,
                             vp(K), vp(V), vp(S), vp(0))


def test_project_validation(L):
    assert _proj(L, D=24) == fl.FLAREPP_UNSUPPORTED
    assert _proj(L, dtype=3) == fl.FLAREPP_UNSUPPORTED
    assert _proj(L, H=17, D=32) == fl.FLAREPP_UNSUPPORTED  # C = 544 > 512
    assert _proj(L, H=9, D=32, dtype=0) == fl.FLAREPP_UNSUPPORTED  # fp32 C = 288 > 256
    assert _proj(L, N=-1) == fl.FLAREPP_INVALID_ARGUMENT
    assert _proj(L, N=(1 << 35) + 1) == fl.FLAREPP_INVALID_ARGUMENT
    assert _proj(L, X=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _proj(L, S=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert _proj(L, Wv=0x3008) == fl.FLAREPP_MISALIGNED
    assert _proj(L, bk=0x5001) == fl.FLAREPP_MISALIGNED  # biases: element alignment
    # Outputs must not overlap the inputs or each other.
    assert _proj(L, K=0x1000 + 32) == fl.FLAREPP_INVALID_ARGUMENT
    assert _proj(L, V=0x7000000 + 64) == fl.FLAREPP_INVALID_ARGUMENT
    assert _proj(L, bk=0x9000000 + 2) == fl.FLAREPP_INVALID_ARGUMENT
    assert _proj(L, N=0) == fl.FLAREPP_OK
    assert _proj(L, H=0) == fl.FLAREPP_OK


def test_out_project_validation(L):
    vp = ctypes.c_void_p
    def call(Y=0x1000, Wo=0x2000, bo=0, H=2, N=64, D=16, dtype=1, out=0x7000000):
        return L.flarepp_out_project(vp(Y), vp(Wo), vp(bo), 1, H, N, D, dtype, vp(out), vp(0))
    assert call(D=8) == fl.FLAREPP_UNSUPPORTED
    assert call(Y=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(out=0x7000008) == fl.FLAREPP_MISALIGNED
    assert call(out=0x1000 + 16) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(N=0) == fl.FLAREPP_OK


def test_block_validation_and_workspace(L):
    vp = ctypes.c_void_p
    def call(X=0x1000, Qs=0x5000, gamma=0x6000, M=8, D=16, H=2, N=64, out=0x7000000, ws=None, ws_bytes=0):
        args = [vp(X), vp(0x10000), vp(0x20000), vp(0x30000), vp(0x40000), vp(0), vp(0), vp(0), vp(0), vp(Qs),
                vp(0x50000), vp(gamma), vp(0), vp(0), 1, H, N, M, D, 1, vp(out)]
        if ws is None:
            return L.flarepp_block(*args, vp(0))
        return L.flarepp_block_ws(*args, vp(ws), ws_bytes, vp(0))
    assert call(M=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(M=513) == fl.FLAREPP_UNSUPPORTED
    assert call(D=24) == fl.FLAREPP_UNSUPPORTED
    assert call(H=17, D=32) == fl.FLAREPP_UNSUPPORTED
    assert call(gamma=0) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(Qs=0x5004) == fl.FLAREPP_MISALIGNED
    assert call(out=0x1000 + 64) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(N=0) == fl.FLAREPP_OK
    need = fl.flarepp_block_workspace_bytes(1, 2, 64, 8, 16, 1)
    assert call(ws=0xF0000000, ws_bytes=need - 1) == fl.FLAREPP_INVALID_ARGUMENT
    assert call(ws=0xF0000010, ws_bytes=need) == fl.FLAREPP_MISALIGNED
    assert fl.flarepp_block_workspace_bytes(1, 2, 64, 0, 16, 1) == 0
    for (B, H, N, M, D, dt) in [(1, 2, 1024, 32, 16, 0), (1, 8, 1 << 20, 512, 32, 1)]:
        es = 2 if dt == 1 else 4
        ws = fl.flarepp_block_workspace_bytes(B, H, N, M, D, dt)
        # The mixer's workspace plus K, V, S and the mixer output, the seeds and the gates.
        assert ws >= fl.flarepp_workspace_bytes(B, H, N, M, D, dt) + 4 * B * H * N * D * es + H * M * D * es
        assert ws < fl.flarepp_workspace_bytes(B, H, N, M, D, dt) + 4 * B * H * N * D * es + H * M * D * es + 2048


def test_microbenchmark_library_loads_and_validates():
    # The roofline microbenchmarks live in a library of their own; invalid sizes are refused before
    # any launch (no GPU needed).
    from rank_latent_routing_amd.build import MB_LIB
    M = ctypes.CDLL(MB_LIB)
    for n in ("flarepp_mb_compute", "flarepp_mb_stream", "flarepp_mb_fanout", "flarepp_mb_kind_name",
              "flarepp_mb_num_kinds"):
        assert hasattr(M, n), n
    M.flarepp_mb_kind_name.restype = ctypes.c_char_p
    kinds = [M.flarepp_mb_kind_name(i).decode() for i in range(M.flarepp_mb_num_kinds())]
    assert kinds[:4] == ["exp", "fma", "exp+fma", "mfma"] and "tile_lds_wg16_sync8_random" in kinds
    assert M.flarepp_mb_kind_name(len(kinds)) is None
    ms = ctypes.c_double()
    vp = ctypes.c_void_p
    assert M.flarepp_mb_compute(0, 0, 16, 1, vp(0x1000), vp(0), ctypes.byref(ms)) != 0
    assert M.flarepp_mb_stream(vp(0x1000), vp(0x2000), ctypes.c_int64(15), 1, 1, vp(0), vp(0), ctypes.byref(ms)) != 0
    M.flarepp_mb_fanout.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                    ctypes.POINTER(ctypes.c_double)]
    assert M.flarepp_mb_fanout(vp(0x1000), vp(0x2000), 15, 1, 1, 1, vp(0), ctypes.byref(ms)) != 0
    assert M.flarepp_mb_fanout(vp(0x1000), vp(0x2000), 16, 5, 1, 1, vp(0), ctypes.byref(ms)) != 0


def _host_inputs(B=1, H=2, N=40, M=8, D=16, dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    big = lambda: torch.zeros((B, H, N, D), dtype=dtype)
    return dict(K=big(), V=big(), S=big(), Qseed=torch.zeros((H, M, D), dtype=dtype),
                Qf=torch.zeros((H, M, D), dtype=dtype), g=torch.zeros(H, dtype=torch.float32))


def test_binding_checks_outputs_before_any_launch():
    # Caller-supplied outputs of the wrong shape, dtype or layout are refused by the binding; every
    # case here raises before the library is asked to launch anything (host tensors, no GPU).
    import torch
    x = _host_inputs()
    bad_out = (torch.zeros((1, 2, 39, 16), dtype=torch.bfloat16), torch.zeros((1, 2, 40, 16), dtype=torch.float32),
               torch.zeros((1, 2, 16, 40), dtype=torch.bfloat16).transpose(2, 3))
    for out in bad_out:
        for fn in (fl.flarepp_mix, fl.flarepp_mix_ws, fl.flarepp_mix_debug):
            with pytest.raises(ValueError, match="out must be"):
                fn(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], out=out)
        with pytest.raises(ValueError, match="out must be"):
            fl.flarepp_flare(x["K"], x["V"], x["Qf"], out=out)
        with pytest.raises(ValueError, match="out must be"):
            fl.flarepp_mix_simplified(x["K"], x["V"], x["S"], x["S"], x["Qseed"], out=out)
    grads = {"dK": torch.zeros_like(x["K"]), "dV": torch.zeros_like(x["K"]), "dS": torch.zeros_like(x["K"]),
             "dQseed": torch.zeros_like(x["Qseed"]), "dQf": torch.zeros_like(x["Qf"]), "dg": torch.zeros(2)}
    dY = torch.zeros_like(x["K"])
    for name, bad in (("dK", torch.zeros((1, 2, 40, 8), dtype=torch.bfloat16)), ("dQf", torch.zeros((2, 8, 16))),
                      ("dg", torch.zeros(3))):
        g2 = dict(grads, **{name: bad})
        with pytest.raises(ValueError, match=name):
            fl.flarepp_mix_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], dY, grads=g2)
    with pytest.raises(ValueError, match="dS"):
        fl.flarepp_mix_backward(x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"], dY,
                                grads={k: v for k, v in grads.items() if k != "dS"})
    # Projections and the block: outputs of the wrong shape.
    X = torch.zeros((1, 40, 32), dtype=torch.bfloat16)
    W = torch.zeros((32, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out K"):
        fl.flarepp_project(X, W, W, W, 2, out=(torch.zeros((1, 2, 40, 8), dtype=torch.bfloat16),) * 3)
    with pytest.raises(ValueError, match="out must be"):
        fl.flarepp_out_project(x["K"], W, out=torch.zeros((1, 40, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        fl.flarepp_block(X, W, W, W, W, x["Qseed"], x["Qf"], torch.zeros(2), out=torch.zeros((1, 41, 32),
                                                                                            dtype=torch.bfloat16))


def test_binding_requires_gpu_tensors_and_a_byte_workspace():
    import torch
    x = _host_inputs()
    args = (x["K"], x["V"], x["S"], x["Qseed"], x["Qf"], x["g"])
    # Host tensors with correct shapes: refused as not on a GPU.
    for fn in (fl.flarepp_mix, fl.flarepp_mix_ws, fl.flarepp_mix_debug):
        with pytest.raises(ValueError, match="GPU"):
            fn(*args)
    with pytest.raises(ValueError, match="GPU"):
        fl.flarepp_flare(x["K"], x["V"], x["Qf"])
    with pytest.raises(ValueError, match="GPU"):
        fl.flarepp_mix_backward(*args, torch.zeros_like(x["K"]))
    with pytest.raises(ValueError, match="GPU"):
        fl.flarepp_mix_simplified(x["K"], x["V"], x["S"], x["S"], x["Qseed"])
    X = torch.zeros((1, 40, 32), dtype=torch.bfloat16)
    W = torch.zeros((32, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fl.flarepp_project(X, W, W, W, 2)
    with pytest.raises(ValueError, match="GPU"):
        fl.flarepp_out_project(x["K"], W)
    with pytest.raises(ValueError, match="GPU"):
        fl.flarepp_block(X, W, W, W, W, x["Qseed"], x["Qf"], torch.zeros(2))
    # A workspace that is not bytes, or not contiguous.
    for ws in (torch.zeros(100, dtype=torch.float32), torch.zeros(200, dtype=torch.uint8)[::2]):
        with pytest.raises(ValueError, match="workspace"):
            fl._require_workspace(ws, torch.device("cpu"))
    with pytest.raises(ValueError, match="workspace must be on"):
        fl._require_workspace(torch.zeros(100, dtype=torch.uint8), torch.device("cuda", 0))


def test_noalloc_rejects_problems_beyond_its_scratch(L):
    # The no-allocation entry point refuses, before touching any device, a problem whose workspace
    # exceeds the static scratch; every benchmark workload fits.
    assert fl.FLAREPP_NOALLOC_SCRATCH_BYTES == 32 << 20
    for shape in ((1, 2, 1024, 32, 16, 0), (4, 8, 16384, 64, 16, 1), (32, 8, 4096, 128, 32, 1),
                  (2, 8, 65536, 256, 32, 1), (1, 8, 1 << 20, 512, 32, 1)):
        assert 0 < fl.flarepp_workspace_bytes(*shape) <= fl.FLAREPP_NOALLOC_SCRATCH_BYTES
    big = (64, 8, 65536, 512, 32, 1)
    assert fl.flarepp_workspace_bytes(*big) > fl.FLAREPP_NOALLOC_SCRATCH_BYTES
    vp = ctypes.c_void_p
    B, H, N, M, D, dt = big
    rc = L.flarepp_mix_noalloc(vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), vp(0x5000), vp(0x6000), B, H,
                               ctypes.c_int64(N), M, D, dt, vp(0x70000000000), vp(0))
    assert rc == fl.FLAREPP_SCRATCH_TOO_SMALL
    assert "scratch" in fl.flarepp_strerror(rc)
    # Validation comes first, as for flarepp_mix.
    assert L.flarepp_mix_noalloc(vp(0), vp(0x2000), vp(0x3000), vp(0x4000), vp(0x5000), vp(0x6000), 1, 1,
                                 ctypes.c_int64(64), 8, 16, 1, vp(0x7000000), vp(0)) == fl.FLAREPP_INVALID_ARGUMENT
    assert L.flarepp_mix_noalloc(vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), vp(0x5000), vp(0x6000), 1, 1,
                                 ctypes.c_int64(0), 8, 16, 1, vp(0x7000000), vp(0)) == fl.FLAREPP_OK
