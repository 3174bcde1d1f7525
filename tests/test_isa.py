"""Checks on the gfx950 assembly of the library's own kernels (built here from source).

* No MFMA has a destination sharing registers with its A or B operand. The double-depth
  v_mfma_f32_16x16x32_bf16 returned wrong products on MI355X when the register allocator placed its
  destination on top of an operand that died at the instruction; the kernels keep such operands
  live past their MFMAs, and this test keeps it that way for every MFMA form.
* Every bf16 dot product that forms a probability's rounding residual (x + hi * -1 + other * 0,
  against a selector held in a register) reads the packed pair converted from that same x. With the
  pair built by a byte permute instead of a packed conversion, the compiler emitted these dot
  products with one pair for every call in some kernels, and the results were wrong.
* No scalar-memory store or atomic (the kernels write only through vector memory).
* No register spills to scratch.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_latent_routing_amd", "csrc")
SOURCES = [os.path.join(CSRC, n) for n in ("kernels.hip", "backward.hip", "project.hip")]


@pytest.fixture(scope="module")
def asm():
    text = []
    with tempfile.TemporaryDirectory() as d:
        for src in SOURCES:
            out = os.path.join(d, os.path.basename(src) + ".s")
            cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-x", "hip", src, "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            text.append(open(out).read())
    return "\n".join(text)


def _regs(tok):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return m.group(1), int(m.group(2)), int(m.group(3))
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return m.group(1), int(m.group(2)), int(m.group(2))
    return None


def test_mfma_destination_never_overlaps_a_or_b(asm):
    kernel, n, bad = None, 0, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            kernel = m.group(1)
            continue
        m = re.match(r"\s*(v_mfma\S*)\s+(\S+),\s*(\S+),\s*(\S+),", line)
        if not m:
            continue
        n += 1
        d, a, b = (_regs(t) for t in m.group(2, 3, 4))
        for src in (a, b):
            if d and src and d[0] == src[0] and not (d[2] < src[1] or src[2] < d[1]):
                bad.append((kernel, line.strip()))
    assert n > 100
    assert not bad, bad[:5]


def test_residual_dot_products_read_their_own_pair(asm):
    defs, sel, n, bad = {}, set(), 0, []
    for line in asm.splitlines():
        if re.match(r"^_Z\S+:", line):
            defs, sel = {}, set()
            continue
        t = line.strip()
        if not t or t.startswith((".", ";")) or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        op, args = parts[0], [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        if op.startswith("v_dot2c_f32_bf16") and len(args) == 3 and args[2] in sel:
            n += 1
            src = defs.get(args[1])
            if src is None or not src[0].startswith("v_cvt_pk_bf16_f32") or args[0] not in src[1][1:]:
                bad.append(t)
        if op.startswith("v_mov_b32") and len(args) == 2 and args[1] in ("0xbf80", "0xffffffffbf800000"):
            sel.add(args[0])
        elif args and re.fullmatch(r"v\d+", args[0]) and op.startswith("v_") and not op.startswith("v_cmp"):
            sel.discard(args[0])
        if args and re.fullmatch(r"v\d+", args[0]) and op.startswith("v_") and not op.startswith("v_cmp"):
            defs[args[0]] = (op, args)
        elif args and re.fullmatch(r"v\[\d+:\d+\]", args[0]):
            r = _regs(args[0])
            for k in range(r[1], r[2] + 1):
                defs.pop(f"v{k}", None)
                sel.discard(f"v{k}")
    assert n > 100
    assert not bad, bad[:5]


def test_no_scalar_memory_writes(asm):
    assert not re.search(r"^\s*s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|dcache_discard)", asm, re.M)


def test_no_scratch_spills(asm):
    sizes = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s*(\d+)", asm)]
    assert sizes and max(sizes) == 0
