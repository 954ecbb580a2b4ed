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


def _kernel_bodies(asm):
    """name -> assembly text of each kernel function."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        out[name] = asm[m.end():end]
    return out


def _innermost_loops(body):
    """Line ranges [header, last back-edge] of the loops that contain no other loop."""
    lines = body.splitlines()
    loops = []
    for n, l in enumerate(lines):
        if "Loop Header" in l and "=>" in l:
            j = n
            while j > 0 and not lines[j].startswith(".LBB"):
                j -= 1
            label = lines[j].split(":")[0]
            ends = [k for k, x in enumerate(lines) if k > j and "branch" in x and x.strip().endswith(label)]
            if ends:                                   # a back edge to the header label
                loops.append((j, max(ends)))
    inner = [(a, b) for (a, b) in loops if not any(a < c and d <= b and (c, d) != (a, b) for (c, d) in loops)]
    return lines, inner


# split_decode_kernel<OUT_F32 = true, FP8 = false, DEV, COMB = true>
_COMBINING_F32_BF16 = re.compile(r"split_decode_kernelILb1ELb0ELb[01]ELb1E")


def test_no_scratch(asm):
    """No kernel touches scratch memory inside a loop over KV blocks (or any innermost loop).  Only
    three kernels use scratch at all, for a few per-piece values (output addresses, bounds) read and
    written outside the block loops: the 128-row kernel (256 accumulation registers hold its
    512 x 32 O^T tile, 128 VGPRs its query rows), at most 128 bytes per lane, the 32-row kernel
    (the same O^T tile, 80 VGPRs of query), at most 256, and the 16-row kernel
    with fp32 output over bf16 rows when it combines split sequences in the same launch (its hot
    loop needs all 512 registers; the write-through partial stores and the combine add a few
    live values), at most 64."""
    sizes = dict(re.findall(r"\.amdhsa_kernel (\S+)\s+\.amdhsa_group_segment_fixed_size \d+\s+"
                            r"\.amdhsa_private_segment_fixed_size (\d+)", asm))
    assert sizes
    for name, size in sizes.items():
        if "wide_decode_kernel" in name:
            assert int(size) <= 128, (name, size)
        elif "split32_decode_kernel" in name:
            assert int(size) <= 256, (name, size)
        elif _COMBINING_F32_BF16.search(name):
            assert int(size) <= 64, (name, size)
        else:
            assert int(size) == 0, (name, size)
    bodies = _kernel_bodies(asm)
    assert any("wide_decode_kernel" in n for n in bodies)
    for name, body in bodies.items():
        lines, inner = _innermost_loops(body)
        for a, b in inner:
            bad = [l for l in lines[a:b + 1] if "scratch_" in l]
            assert not bad, (name, bad[:3])
