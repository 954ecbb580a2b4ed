"""Static checks on the gfx950 assembly of the kernels (CPU only; needs hipcc).

- Runs of consecutive LDS reads: no read's destination registers may be an address
  register of a later read in the same run (a returning read would clobber the address
  before it is used).  The compiler schedules these reads; the check guards the inline
  asm around them (DMA blocks, explicit waits) against upsetting that.
- No scalar-memory stores or atomics anywhere; every kernel runs without scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

from mla_decode_attention_paged_amd import build as mbuild

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "mla_kernels.s"
    src = os.path.join(mbuild.CSRC, "mla_kernels.hip")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", mbuild.INCLUDE, "-I", mbuild.CSRC, src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def test_lds_read_batches_do_not_clobber_their_addresses(asm):
    lines = [l.split() for l in asm.splitlines()]
    batches = overlaps = 0
    i = 0
    while i < len(lines):
        if lines[i] and lines[i][0].startswith("ds_read"):
            j = i
            while j < len(lines) and lines[j] and lines[j][0].startswith("ds_read"):
                j += 1
            batch = lines[i:j]
            batches += 1
            for a in range(len(batch)):
                dst = _regs(batch[a][1].rstrip(","))
                for b in range(a + 1, len(batch)):
                    if dst & _regs(batch[b][2].rstrip(",")):
                        overlaps += 1
            i = j
        else:
            i += 1
    assert batches > 20
    assert overlaps == 0


def test_no_scalar_memory_writes(asm):
    bad = [l for l in asm.splitlines() if re.match(r"\s*s_(atomic|store|buffer_store|buffer_atomic|dcache_wb|dcache_discard)", l)]
    assert not bad, bad[:5]


def test_no_scratch(asm):
    sizes = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", asm)]
    assert sizes and max(sizes) == 0
