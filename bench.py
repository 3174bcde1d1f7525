"""Throughput of the FLARE++ mixer forward pass on one MI355X.

A step is one full mixer call (synthesis, gate, encode, decode over every (b, h)) on the
million-token workload: B=1, H=8, N=2^20 tokens on a random closed surface, M=512 latents, D=32,
bf16 inputs with fp32 accumulation, inputs resident in HBM. The JSON line reports tokens*heads/s,
the achieved TFLOP/s (12 N M D flops per head), per-kernel event timings, the roofline position of
the dominant kernel and the float64 CPU oracle timed on a bounded sample of the same workload.

Plain FLARE and simplified FLARE++ on the same workload ("variants"), the backward pass
(flarepp_mix_backward with a seeded output cotangent, the forward recomputed inside it; "backward")
and the whole block (flarepp_block: projections of a seeded input X [B, N, H D] with the pages'
near-identity weights, the mixer, the output projection; "block") are timed afterwards, each in a
region of its own.

"shard" times one GPU's share of the same workload split over 8 GPUs by token ranges (the pages'
context parallelism): the first N/8 tokens of every (b, h) slice through the same call.

Per call the line also gives the median and minimum of the K timed calls; `graph_replay` the time
per call when the call, captured once in a HIP graph, is replayed K times (the host out of the
launch chain; `value` stays the eager call); `--cold` adds the median and minimum for calls that
each follow a 1 GiB write (the smaller workloads' inputs otherwise stay in the 256 MB MALL between
calls).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..5] [--no-cpu-baseline]
                      [--cpu-sample-heads H] [--copy-calibration] [--no-backward] [--no-variants]
                      [--no-block] [--no-shard] [--no-graph] [--cold]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense).
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# v_exp_f32 rate of the whole chip, measured by the exp microbenchmark (bench.py --microbench, summary
# in profiles/roofline_microbenchmarks.md): 1.46e13 exponentials per second, 4.49 ns per wave
# instruction on a SIMD.
PEAK_EXP_PER_S = 1.46e13

KERNELS = ["synthesis_partial", "merge_gate", "encode_partial", "merge", "decode"]
# Backward kernels (flarepp_mix_backward) and the recomputed forward kernels it launches.
BWD_KERNELS = ["synthesis_partial", "merge_gate", "encode_partial", "merge", "bwd_center", "bwd_token_decode",
               "bwd_latent_decode", "bwd_reduce_decode", "bwd_latent_encode", "bwd_reduce_gate",
               "bwd_latent_synthesis", "bwd_reduce_synthesis", "bwd_token_encode", "bwd_token_synthesis"]
# Algorithmic flops per (token, latent) pair per D of each backward kernel, counting each distinct
# product of the method once (the hi/lo operand pairs are not counted): scores and dP recomputed
# where a kernel needs them, and the products it accumulates.
BWD_FLOPS_PER_NMD = {"synthesis_partial": 4, "encode_partial": 4, "bwd_token_decode": 10, "bwd_latent_decode": 8,
                     "bwd_latent_encode": 6, "bwd_latent_synthesis": 6, "bwd_token_encode": 8,
                     "bwd_token_synthesis": 8}
# The forward kernels' sources, in the order their bytes enter the profile's fingerprint.
KERNEL_SRCS = [os.path.join(ROOT, "rank_latent_routing_amd", "csrc", n) for n in ("kernels.hip", "device.h")]
PROFILE = os.path.join(ROOT, "profiles", "flarepp_mixer_1M_tokens.md")
# The backward kernels' sources (with the forward's, whose hi/lo instance the recompute runs) and the
# backward's kernel-trace summary.
BWD_SRCS = [os.path.join(ROOT, "rank_latent_routing_amd", "csrc", n) for n in ("backward.hip", "kernels.hip", "device.h")]
BWD_PROFILE = os.path.join(ROOT, "profiles", "flarepp_mixer_backward_1M_tokens.md")
# The projection kernel's sources and the block's counter summary.
PROJECT_SRCS = [os.path.join(ROOT, "rank_latent_routing_amd", "csrc", n) for n in ("project.hip", "device.h")]
BLOCK_PROFILE = os.path.join(ROOT, "profiles", "flarepp_block_1M_tokens.md")


def _code_only(text):
    """Source text with // and /* */ comments and trailing blanks removed: a comment edit leaves the
    compiled kernels, and so a profile taken on them, unchanged."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_source_hash(srcs=None):
    """sha256 over the code of kernel sources, comments removed (default: the forward's, kernels.hip
    then device.h)."""
    import hashlib
    h = hashlib.sha256()
    for src in srcs or KERNEL_SRCS:
        with open(src, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def profiled_traffic(kernel, profile=PROFILE, key="forward_sources_sha256", srcs=None):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter summary: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by the factors a 256 MiB device copy measured in the same
    runs. None when the summary is missing or was taken on a different kernel source."""
    try:
        lines = open(profile).read().splitlines()
    except OSError:
        return None
    rec = None
    for ln in lines:
        if ln.startswith("traffic-json: "):
            rec = json.loads(ln[len("traffic-json: "):])
    if not rec or rec.get(key) != kernel_source_hash(srcs):
        return None
    k = rec.get("per_launch_bytes", {}).get(kernel)
    return None if k is None else float(k)


def profiled_kernel_us(kernel, profile=PROFILE, key="forward_sources_sha256", srcs=None):
    """Average dispatch duration (us) of `kernel` in a committed rocprofv3 kernel trace, or None when
    the summary is missing or was taken on a different kernel source."""
    try:
        lines = open(profile).read().splitlines()
    except OSError:
        return None
    rec = None
    for ln in lines:
        if ln.startswith("traffic-json: "):
            rec = json.loads(ln[len("traffic-json: "):])
    if not rec or rec.get(key) != kernel_source_hash(srcs):
        return None
    v = rec.get("kernel_avg_us", {}).get(kernel)
    return None if v is None else float(v)


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=8,
                    help="(b, h) slices of the workload the CPU baseline runs (default 8: all of the 1M-token one)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-variants", action="store_true", help="skip plain FLARE and simplified FLARE++")
    ap.add_argument("--no-block", action="store_true", help="skip the block (projections + mixer + output projection)")
    ap.add_argument("--no-shard", action="store_true", help="skip one GPU's share of an 8-way token split")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the mixer call")
    ap.add_argument("--cold", action="store_true",
                    help="also time K calls with a 1 GiB write between them (inputs out of the caches)")
    ap.add_argument("--microbench", action="store_true",
                    help="also run the roofline microbenchmarks (exp, fp32 FMA and bf16 MFMA issue rates, their "
                         "mixes, the partial kernels' tile loop in isolation, HBM read and copy rates) into a 'microbench' field")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device-to-device copy before the timed region (a reference "
                         "dispatch for scaling the HBM byte counters of a profile)")
    return ap.parse_args()


def kernel_flops(name, w):
    """Algorithmic flops of one launch: each of the three routing calls costs 4 N M D per (b, h)
    (2 for the scores, 2 for the probabilities times values); merges are not counted."""
    per = 4.0 * w.N * w.M * w.D * w.B * w.H
    return per if name in ("synthesis_partial", "encode_partial", "decode") else 0.0


def kernel_bytes(name, w):
    """Algorithmic HBM bytes of one launch: the token tensors it must read or write once (K, V, S,
    out at the input width) and, for decode, the latent tensors c*Q and Z it reads; the fp32 chunk
    partials of the split-N kernels (under 4% of their bytes here) are not counted."""
    es = 2 if w.dtype == "bf16" else 4
    tok = float(w.N) * w.D * w.B * w.H * es
    lat = float(w.M) * w.D * w.B * w.H
    if name == "synthesis_partial":
        return tok
    if name == "encode_partial":
        return 2 * tok
    if name == "decode":
        return 2 * tok + lat * (es * 3 + es)
    return 0.0


def cpu_baseline(w, heads):
    """The float64 oracle, as it stands, on the first `heads` (b, h) slices of the same workload (all N
    tokens each), one slice per worker thread over the host's cores: numpy releases the interpreter
    lock in its BLAS products and elementwise exponentials, and the BLAS threads are divided among
    the workers so that the threads in use match the cores."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from workloads import to_float64
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    slices = [(b, h) for b in range(w.B) for h in range(w.H)][:max(1, heads)]
    workers = min(len(slices), cores)
    blas = max(1, cores // workers)

    def run(bh):
        b, h = bh
        oracle.mix_head(to_float64(w.K[b, h], w.dtype), to_float64(w.V[b, h], w.dtype),
                        to_float64(w.S[b, h], w.dtype), to_float64(w.Qseed[h], w.dtype),
                        to_float64(w.Qf[h], w.dtype), float(w.g[h]), block=65536)

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=blas)
    except Exception:  # noqa: BLE001
        limit, blas = None, 1
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(run, slices))
    dt = time.perf_counter() - t0
    if limit is not None:
        limit.restore_original_limits()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": len(slices) * w.N / dt, "unit": "tokens*heads/s", "cores": workers * blas, "kind": "oracle",
            "sample": f"{len(slices)} of {w.B * w.H} (b, h) slices, all {w.N} tokens each, M={w.M}, D={w.D}, "
                      f"float64 numpy oracle; {dt:.2f} s wall; {workers} worker threads (one slice each) x "
                      f"{blas} BLAS threads",
            "host_logical_cpus": os.cpu_count(), "cpu_model": model}


def microbench():
    """The denominators of the rooflines, measured: the issue rate of v_exp_f32, of fp32 FMAs and of
    32x32x16 bf16 MFMAs, alone and mixed (a mix that takes about as long as its slower part alone
    shows that the two pipes overlap), at 4 waves per SIMD on every SIMD of the chip; the partial
    kernels' tile loop in isolation (register forms, LDS operands, 16-wave workgroups, a barrier
    every 8 tiles); and HBM read and copy bandwidth over 2 GiB. Rates are per second over the whole
    device; times per wave instruction are per SIMD."""
    import ctypes

    import torch

    from rank_latent_routing_amd.build import MB_LIB
    if not os.path.exists(MB_LIB):
        raise RuntimeError(f"{MB_LIB} is missing: build it with `python -m rank_latent_routing_amd.build`")
    L = ctypes.CDLL(MB_LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.flarepp_mb_compute.argtypes = [i32, i32, i32, i32, vp, vp, ctypes.POINTER(ctypes.c_double)]
    L.flarepp_mb_compute.restype = i32
    L.flarepp_mb_stream.argtypes = [vp, vp, i64, i32, i32, vp, vp, ctypes.POINTER(ctypes.c_double)]
    L.flarepp_mb_stream.restype = i32
    L.flarepp_mb_fanout.argtypes = [vp, vp, i64, i32, i32, i32, vp, ctypes.POINTER(ctypes.c_double)]
    L.flarepp_mb_fanout.restype = i32
    L.flarepp_mb_kind_name.argtypes = [i32]
    L.flarepp_mb_kind_name.restype = ctypes.c_char_p
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    wps = 4
    grid = cus * 4 * wps // 4
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    iters = 4096
    # Per loop iteration and lane: (exps, fmas, MFMAs) of each kind, in the library's order.
    work = {"exp": (8, 0, 0), "fma": (0, 8, 0), "exp+fma": (8, 8, 0), "mfma": (0, 0, 4), "mfma+fma": (0, 32, 4),
            "mfma+exp": (16, 0, 4), "mfma+exp+fma": (16, 16, 4), "tile": (16, 0, 0), "tile_agpr_acc": (16, 0, 0),
            "tile_lds": (16, 0, 0), "tile_lds_wg16": (16, 0, 0), "tile_lds_wg16_sync8": (16, 0, 0),
            "tile_lds_wg16_sync8_random": (16, 0, 0), "exp_f16": (8, 0, 0), "tile_random_no_row_sums": (16, 0, 0),
            "tile_random_dot2_row_sums": (16, 0, 0), "mfma_random": (0, 0, 4)}
    res = {"cus": cus, "waves_per_simd": wps, "iters": iters, "kinds": {}}
    lanes = grid * 256
    waves = grid * 4
    for k in range(len(work)):
        name = L.flarepp_mb_kind_name(k).decode()
        ms = ctypes.c_double()
        rc = L.flarepp_mb_compute(k, grid, iters, 5, ctypes.c_void_p(out.data_ptr()), stream, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"microbenchmark {name}: HIP error {rc}")
        t = ms.value * 1e-3
        ne, nf, nm = work[name]
        # Time per wave instruction on one SIMD: launch time over the instructions each SIMD issues.
        rec = {"ms": round(ms.value, 4)}
        if ne:
            rec["exp_per_s"] = lanes * iters * ne / t
            rec["ns_per_wave_exp"] = round(t * 1e9 / (iters * ne * wps), 3)
        if nf:
            rec["fma_per_s"] = lanes * iters * nf / t
            rec["ns_per_wave_fma"] = round(t * 1e9 / (iters * nf * wps), 3)
        if nm:
            rec["mfma_tflops"] = round(waves * iters * nm * 32 * 32 * 16 * 2 / t * 1e-12, 1)
        if name.startswith("tile"):
            # One 32x32 score tile per wave and iteration: time per tile on one SIMD.
            rec["ns_per_tile_per_simd"] = round(t * 1e9 / (iters * wps), 2)
        res["kinds"][name] = rec
    del out
    nbytes = 2 ** 31
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    sgrid = cus * 8
    red = torch.empty(sgrid * 256, dtype=torch.float32, device="cuda")
    for name, d, moved in (("hbm_read", None, nbytes), ("hbm_copy", dst, 2 * nbytes)):
        ms = ctypes.c_double()
        rc = L.flarepp_mb_stream(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(0 if d is None else d.data_ptr()),
                                 nbytes, sgrid, 5, ctypes.c_void_p(red.data_ptr()), stream, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"microbenchmark {name}: HIP error {rc}")
        res[name + "_gbs"] = round(moved / (ms.value * 1e-3) * 1e-9, 1)
    # Writes alone, and the front projection's mix: one tensor read, three of its size written.
    del dst
    nfan = 2 ** 29
    fdst = torch.empty(3 * nfan // 4, dtype=torch.float32, device="cuda")
    for name, s_ptr, copies, moved in (("hbm_write", 0, 1, nfan), ("hbm_read1_write3", src.data_ptr(), 3, 4 * nfan)):
        ms = ctypes.c_double()
        rc = L.flarepp_mb_fanout(ctypes.c_void_p(s_ptr), ctypes.c_void_p(fdst.data_ptr()), nfan, copies, sgrid, 5,
                                 stream, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"microbenchmark {name}: HIP error {rc}")
        res[name + "_gbs"] = round(moved / (ms.value * 1e-3) * 1e-9, 1)
    return res


def _kernel_times(steps, call):
    """K more calls with the library's event pairs around each kernel: {kernel: ms per launch}."""
    import torch

    import rank_latent_routing_amd as fl
    fl.flarepp_timing_enable(True)
    fl.flarepp_timing_read()
    torch.cuda.synchronize()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    fl.flarepp_timing_enable(False)
    return {k: v[0] / max(v[1], 1) for k, v in fl.flarepp_timing_read().items()}


def _time_steps(args, call):
    """Warm-up, then K calls in a region bracketed by synchronizations, timed with HIP events on the
    current stream and the wall clock; returns ms per call."""
    import torch
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    return max(ev0.elapsed_time(ev1), (time.perf_counter() - t0) * 1e3) / args.steps


def _graph_replay(args, call, stream):
    """The call captured once in a HIP graph and replayed K times: ms per replay."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        g.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph = {"ms_per_step": g0.elapsed_time(g1) / args.steps, "calls": args.steps}
    del g
    return graph


def variants(args, w, dev, dt_code):
    """Plain FLARE (Eq. 3, the fixed queries Qf used as given) and simplified FLARE++ (Eq. 20, S as
    the synthesis keys and seeded separate synthesis values) on the same workload."""
    import numpy as np
    import torch

    import rank_latent_routing_amd as fl
    from workloads import make_synthesis_values

    sv = np.ascontiguousarray(make_synthesis_values(w))
    Sv = (torch.from_numpy(sv.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" else torch.from_numpy(sv)).cuda()
    out = torch.empty_like(dev["K"])
    ws = torch.empty(fl.flarepp_workspace_bytes(w.B, w.H, w.N, w.M, w.D, dt_code), dtype=torch.uint8, device="cuda")
    res = {}
    for name, call in (
            ("flare", lambda: fl.flarepp_flare(dev["K"], dev["V"], dev["Qf"], out=out, workspace=ws)),
            ("simplified", lambda: fl.flarepp_mix_simplified(dev["K"], dev["V"], dev["S"], Sv, dev["Qseed"], out=out,
                                                             workspace=ws))):
        ms = _time_steps(args, call)
        res[name] = {"ms_per_step": ms, "value": w.B * w.H * w.N / (ms * 1e-3), "unit": "tokens*heads/s"}
    return res


def shard(args, w, dev, dt_code, ranks=8):
    """One GPU's share of the workload split over `ranks` GPUs by token ranges (context parallelism,
    Appendix B): the first N / ranks tokens of every (b, h) slice through the same mixer call. Under
    that split each GPU runs the partial kernels and the decode on its own tokens; what this figure
    leaves out is the exchange of the latent partials between GPUs (one all-gather of M (D + 2)
    values per head and routing call) and the merge of the gathered sets."""
    import torch

    import rank_latent_routing_amd as fl
    n = w.N // ranks
    K, V, S = (dev[k][:, :, :n].contiguous() for k in ("K", "V", "S"))
    out = torch.empty_like(K)
    ws = torch.empty(fl.flarepp_workspace_bytes(w.B, w.H, n, w.M, w.D, dt_code), dtype=torch.uint8, device="cuda")
    call = lambda: fl.flarepp_mix_ws(K, V, S, dev["Qseed"], dev["Qf"], dev["g"], out=out, workspace=ws)
    ms = _time_steps(args, call)
    kern = _kernel_times(args.steps, call)
    return {"ranks": ranks, "N": n, "ms_per_step": ms, "value": w.B * w.H * n / (ms * 1e-3),
            "unit": "tokens*heads/s", "kernels": {k: round(v, 4) for k, v in kern.items() if v > 0}}


def backward(args, w, dev, dt_code, peak):
    """The mixer's backward pass (flarepp_mix_backward, forward recomputed inside) on the same inputs
    with a seeded cotangent dY, timed like the forward in a region of its own; then a training step's
    two calls, flarepp_mix_forward_saved and flarepp_mix_backward_saved (no recompute), each timed on
    its own ("saved")."""
    import numpy as np
    import torch

    import rank_latent_routing_amd as fl
    from workloads import make_cotangent

    dy = np.ascontiguousarray(make_cotangent(w))
    dY = (torch.from_numpy(dy.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" else torch.from_numpy(dy)).cuda()
    grads = {k: torch.empty_like(dev[src]) for k, src in (("dK", "K"), ("dV", "K"), ("dS", "K"), ("dQseed", "Qseed"),
                                                           ("dQf", "Qf"), ("dg", "g"))}
    ws = torch.empty(fl.flarepp_backward_workspace_bytes(w.B, w.H, w.N, w.M, w.D, dt_code), dtype=torch.uint8,
                     device="cuda")
    call = lambda: fl.flarepp_mix_backward(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"], dY,
                                           grads=grads, workspace=ws)
    ms = _time_steps(args, call)
    # Per-kernel durations from K more calls (events between the kernels stay out of the step time).
    per_kernel = _kernel_times(args.steps, call)
    kern = {k: per_kernel[k] for k in BWD_KERNELS}
    nmd = float(w.N) * w.M * w.D * w.B * w.H
    dom = max(kern, key=kern.get)
    dom_flops = BWD_FLOPS_PER_NMD.get(dom, 0) * nmd
    achieved = dom_flops / (kern[dom] * 1e-3) * 1e-12
    prof_us = profiled_kernel_us(dom, BWD_PROFILE, "backward_sources_sha256", BWD_SRCS) if args.config == 5 else None
    # A training step's two calls: the forward that keeps the backward's starting state, then the
    # backward from it (no recompute).
    out = torch.empty_like(dev["K"])
    ws_saved = torch.empty_like(ws)
    fwd_saved = lambda: fl.flarepp_mix_forward_saved(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"],
                                                     workspace=ws_saved, out=out)
    bwd_saved = lambda: fl.flarepp_mix_backward_saved(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"],
                                                      dev["g"], dY, workspace=ws_saved, grads=grads)
    ms_fs = _time_steps(args, fwd_saved)
    ms_bs = _time_steps(args, bwd_saved)
    saved_kern = _kernel_times(args.steps, bwd_saved)
    return {"ms_per_step": ms, "value": w.B * w.H * w.N / (ms * 1e-3), "unit": "tokens*heads/s",
            "algorithmic_tflops": sum(BWD_FLOPS_PER_NMD.values()) * nmd / (ms * 1e-3) * 1e-12,
            "kernels": {k: round(v, 4) for k, v in kern.items()},
            "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "kernel_ms": round(kern[dom], 4),
                         "flops_per_launch": dom_flops, "profile_kernel_us": prof_us,
                         "frac_profile": (round(dom_flops / (prof_us * 1e-6) * 1e-12 / peak, 4) if prof_us else None)},
            "saved": {"forward_ms": ms_fs, "backward_ms": ms_bs, "training_step_ms": ms_fs + ms_bs,
                      "backward_value": w.B * w.H * w.N / (ms_bs * 1e-3),
                      "kernels": {k: round(v, 4) for k, v in saved_kern.items() if v > 0}}}


BLOCK_KERNELS = ["block_params", "project", "synthesis_partial", "merge_gate", "encode_partial", "merge", "decode",
                 "out_project"]


def block(args, w, dt_code):
    """The block (flarepp_block_ws) on a seeded input X of the workload's shape and family with the
    pages' near-identity projection weights: per-kernel event timings, and the projection kernels'
    position against the HBM roofline on their algorithmic bytes (X read once, K, V, S written once,
    the weights read once; the output projection: Y read once, out written once)."""
    import numpy as np
    import torch

    import rank_latent_routing_amd as fl
    from workloads import make_block_inputs

    bi = make_block_inputs(w, init="identity")

    def dev(arr, transpose=False):
        a = np.ascontiguousarray(arr.T if transpose else arr)
        return (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" else torch.from_numpy(a)).cuda()

    X = dev(bi.X)
    Wk, Wv, Ws, Wo = (dev(m, True) for m in (bi.Wk, bi.Wv, bi.Ws, bi.Wo))
    bk, bv, bs, bo, nq, nk = (dev(v) for v in (bi.bk, bi.bv, bi.bs, bi.bo, bi.nq, bi.nk))
    Qs, Qf = dev(w.Qseed), dev(w.Qf)
    gamma = torch.from_numpy(bi.gamma).cuda()
    out = torch.empty_like(X)
    ws = torch.empty(fl.flarepp_block_workspace_bytes(w.B, w.H, w.N, w.M, w.D, dt_code), dtype=torch.uint8,
                     device="cuda")
    del bi
    call = lambda: fl.flarepp_block(X, Wk, Wv, Ws, Wo, Qs, Qf, gamma, bk=bk, bv=bv, bs=bs, bo=bo, nq=nq, nk=nk,
                                    out=out, workspace=ws)
    ms = _time_steps(args, call)
    per_kernel = _kernel_times(args.steps, call)
    kern = {k: per_kernel[k] for k in BLOCK_KERNELS}
    es = 2 if w.dtype == "bf16" else 4
    C = w.H * w.D
    big = float(w.B) * w.N * C * es
    proj_bytes = 4 * big + 3 * C * C * es
    outp_bytes = 2 * big + C * C * es
    proj_flops = 2.0 * w.B * w.N * C * 3 * C
    gbs = proj_bytes / (kern["project"] * 1e-3) * 1e-9
    return {"ms_per_step": ms, "value": w.B * w.H * w.N / (ms * 1e-3), "unit": "tokens*heads/s",
            "kernels": {k: round(v, 4) for k, v in kern.items()},
            "project_roofline": {"bound": "hbm", "kernel": "project", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                 "traffic": profiled_traffic("project", BLOCK_PROFILE, "project_sources_sha256",
                                                             PROJECT_SRCS) if args.config == 5 else None,
                                 "algorithmic_bytes_per_launch": proj_bytes, "kernel_ms": round(kern["project"], 4),
                                 "mfma_tflops": round(proj_flops / (kern["project"] * 1e-3) * 1e-12, 1)},
            "out_project_gbs": round(outp_bytes / (kern["out_project"] * 1e-3) * 1e-9, 1)}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (the mixer would shard "
              "over (b, h) or over token ranges with a log-sum-exp merge of the latent partials); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rank_latent_routing_amd as fl
    from workloads import DESCRIPTIONS, FAMILIES, make_workload

    fl.lib()
    w = make_workload(args.config)
    dev = {}
    for name in ("K", "V", "S", "Qseed", "Qf"):
        arr = np.ascontiguousarray(getattr(w, name))
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" else torch.from_numpy(arr)
        dev[name] = t.cuda()
    dev["g"] = torch.from_numpy(w.g).cuda()
    out = torch.empty_like(dev["K"])
    dt_code = fl.FLAREPP_BF16 if w.dtype == "bf16" else fl.FLAREPP_FP32
    ws = torch.empty(fl.flarepp_workspace_bytes(w.B, w.H, w.N, w.M, w.D, dt_code), dtype=torch.uint8, device="cuda")
    call = lambda: fl.flarepp_mix_ws(dev["K"], dev["V"], dev["S"], dev["Qseed"], dev["Qf"], dev["g"], out=out,
                                     workspace=ws)

    if args.copy_calibration:
        src = torch.empty(64 * 2 ** 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # Timed region: K steps bracketed by synchronizations, one HIP event on the library's stream
    # after each step (the step durations) and the wall clock around the whole region.
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        call()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = max(dev_ms, wall * 1e3) / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))

    # The same K steps again with the library's event pairs around each kernel (per-kernel
    # durations for the roofline). Kept out of the region above: at the small workloads the
    # events between kernels would add a visible share of each step.
    per_kernel = _kernel_times(args.steps, call)

    # The same call captured once in a HIP graph and replayed K times (the workspace entry point
    # enqueues kernels only): what remains of the launch chain's gaps when the host is out of it.
    graph = None
    if not args.no_graph:
        try:
            graph = _graph_replay(args, call, stream)
        except Exception as e:  # noqa: BLE001
            import traceback
            traceback.print_exc()
            graph = {"error": f"{type(e).__name__}: {e}"[:300]}

    cold = None
    if args.cold:
        # Each timed call follows a 1 GiB write, which evicts the inputs from L2 and the MALL.
        flush = torch.empty(2 ** 28, dtype=torch.float32, device="cuda")
        cms = []
        for _ in range(args.steps):
            flush.fill_(1.0)
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            call()
            a1.record(stream)
            torch.cuda.synchronize()
            cms.append(a0.elapsed_time(a1))
        cms.sort()
        cold = {"ms_median": cms[len(cms) // 2], "ms_min": cms[0], "flush_bytes": 2 ** 30, "calls": len(cms)}
        del flush

    tok_heads = w.B * w.H * w.N
    value = tok_heads / (ms_per_step * 1e-3)
    flops = 12.0 * w.N * w.M * w.D * w.B * w.H
    exps = 3.0 * w.N * w.M * w.B * w.H
    es = 2 if w.dtype == "bf16" else 4
    hbm_bytes = 5.0 * w.N * w.D * w.B * w.H * es + 2.0 * w.H * w.M * w.D * es
    tflops = flops / (ms_per_step * 1e-3) * 1e-12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS

    kern = {k: {"ms_avg": per_kernel[k]} for k in KERNELS}
    dom = max(KERNELS, key=lambda k: kern[k]["ms_avg"])
    dom_ms = kern[dom]["ms_avg"]
    achieved = kernel_flops(dom, w) / (dom_ms * 1e-3) * 1e-12
    traffic = profiled_traffic(dom) if args.config == 5 else None
    # The same kernel's average duration in the committed kernel trace (same sources), for a fraction
    # that can be recomputed from the profile alone.
    prof_us = profiled_kernel_us(dom) if args.config == 5 else None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "profile_kernel_us": prof_us,
                "frac_profile": (round(kernel_flops(dom, w) / (prof_us * 1e-6) * 1e-12 / peak, 4)
                                 if prof_us else None),
                "kernel_ms": round(dom_ms, 4), "flops_per_launch": kernel_flops(dom, w),
                "algorithmic_bytes_per_launch": kernel_bytes(dom, w),
                "hbm_gbs": round(kernel_bytes(dom, w) / (dom_ms * 1e-3) * 1e-9, 1),
                "exp_frac": round((w.N * w.M * w.B * w.H) / (dom_ms * 1e-3) / PEAK_EXP_PER_S, 4)}

    res = {
        "metric": "FLARE++ mixer tokens*heads/s (N=1M, M=512)",
        "value": value,
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_median": step_ms[len(step_ms) // 2],
        "ms_min": step_ms[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"FLARE++ mixer forward: {DESCRIPTIONS[args.config]}", "B": w.B, "H": w.H, "N": w.N,
                   "M": w.M, "D": w.D, "inputs": FAMILIES[w.kind]},
        "tflops": tflops,
        "mfma_frac": tflops / peak,
        "hbm_frac": hbm_bytes / (ms_per_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "exp_frac": exps / (ms_per_step * 1e-3) / PEAK_EXP_PER_S,
        "kernels": {k: round(v["ms_avg"], 4) for k, v in kern.items()},
        "roofline": roofline,
    }
    if cold is not None:
        res["cold"] = cold
    if graph is not None:
        res["graph_replay"] = graph

    def leg(name, fn, *a):
        # An extra leg that fails is reported in its field (traceback on stderr) and does not take
        # the headline measurement above with it.
        try:
            res[name] = fn(*a)
        except Exception as e:  # noqa: BLE001
            import traceback
            traceback.print_exc()
            res[name] = {"error": f"{type(e).__name__}: {e}"[:300]}

    if not args.no_variants:
        leg("variants", variants, args, w, dev, dt_code)
    if not args.no_shard:
        leg("shard", shard, args, w, dev, dt_code)
    if not args.no_backward:
        leg("backward", backward, args, w, dev, dt_code, peak)
    if not args.no_block:
        leg("block", block, args, w, dt_code)
    if args.microbench:
        leg("microbench", microbench)
    if not args.no_cpu_baseline:
        leg("cpu_baseline", cpu_baseline, w, args.cpu_sample_heads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
