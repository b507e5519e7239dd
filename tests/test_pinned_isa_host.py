"""The 4-wave 256-tile kernels keep their accumulators in fixed AGPRs and
schedule their own waits; both rest on what the compiler emits, so this test
compiles ns_kernels.hip for gfx950 to assembly (with the library's own flags)
and checks every ns_pinned_kernel instantiation:

- no scratch memory, and arch VGPRs + the 256 pinned AGPRs within the 512 a
  lane has at one wave per SIMD;
- the AGPRs are touched only by the kernel's own MFMAs, zeroing, initial
  writes and reads: no v_accvgpr_mov, and exactly 256 v_accvgpr_read and 256
  v_accvgpr_write per instantiation;
- each main loop (two K stages per iteration) holds exactly two
  ``s_waitcnt vmcnt``, the schedule's own (one per stage, before its barrier):
  a compiler-inserted wait for the direct-to-LDS loads in flight would
  serialise the operand loads with the MFMAs.

No GPU is needed (hipcc cross-compiles)."""

import os
import re
import shutil
import subprocess

import pytest

from newton_schulz_quintic_amd import build as nsq_build

SRC = os.path.join(nsq_build.CSRC, "ns_kernels.hip")


def _kernels(asm: str):
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_ZN\w+):", asm, re.M)]
    for k, (pos, name) in enumerate(starts):
        end = starts[k + 1][0] if k + 1 < len(starts) else len(asm)
        if "ns_pinned_kernel" in name:
            yield name, asm[pos:end].splitlines()


def _dma_loops(lines):
    for i, line in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):.*Loop Header", line)
        if not m:
            continue
        back = re.compile(r"s_cbranch_\w+ " + re.escape(m.group(1)) + r"$")
        j = next((j for j in range(i + 1, len(lines)) if back.search(lines[j].strip())), None)
        if j is None:
            continue
        body = lines[i:j + 1]
        if any("buffer_load" in x and " lds" in x for x in body):
            yield m.group(1), body


@pytest.mark.skipif(not os.path.exists(nsq_build._hipcc()), reason="hipcc not found")
def test_pinned_kernels_isa(tmp_path):
    out = str(tmp_path / "ns_kernels.s")
    cmd = ([nsq_build._hipcc()] + nsq_build.COMMON + nsq_build.DEVICE
           + ["--cuda-device-only", "-S", SRC, "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asm = open(out).read()
    found = 0
    for name, lines in _kernels(asm):
        found += 1
        text = "\n".join(lines)
        count = lambda pat: len(re.findall(pat, text))
        assert count(r"scratch_(load|store)") == 0, name
        nv = int(re.search(r"; NumVgprs: (\d+)", text).group(1))
        na = int(re.search(r"; NumAgprs: (\d+)", text).group(1))
        assert na == 256 and nv + na <= 512, (name, nv, na)
        assert count(r"\bv_accvgpr_mov") == 0, name
        assert count(r"\bv_accvgpr_read") == 256, name
        assert count(r"\bv_accvgpr_write") == 256, name
        loops = list(_dma_loops(lines))
        assert loops, name
        for label, body in loops:
            waits = sum("s_waitcnt" in x and "vmcnt" in x for x in body)
            assert waits == 2, (name, label, waits)
    assert found == 4
    for m in re.finditer(r"\.name:\s+(\S*ns_pinned_kernel\S*)", asm):
        size = re.compile(r"\.private_segment_fixed_size:\s+(\d+)").search(asm, m.end())
        assert size and int(size.group(1)) == 0, m.group(1)
