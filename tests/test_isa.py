"""Checks on the gfx950 assembly of the library's own kernels (built here from source).

* No MFMA has a destination sharing registers with its A or B operand. The double-depth
  v_mfma_f32_16x16x32_bf16 returned wrong products on MI355X when the register allocator placed its
  destination on top of an operand that died at the instruction; the kernels keep such operands
  live past their MFMAs, and this test keeps it that way for every MFMA form.
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


def test_no_scalar_memory_writes(asm):
    assert not re.search(r"^\s*s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|dcache_discard)", asm, re.M)


def test_no_scratch_spills(asm):
    sizes = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s*(\d+)", asm)]
    assert sizes and max(sizes) == 0
