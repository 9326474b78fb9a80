"""No MFMA result of the library's kernels is read through a branch before
its passes have retired, and no kernel spills registers to scratch (CPU:
compiles every source to gfx950 assembly).

The bf16 backward row pass once gave wrong weight-gradient columns 3, 7, 11
and 15 (accumulator element 3 of the first row tile) when its column-tile
loop was cut short at run time: the compiled code branched from the MFMA
pair writing that accumulator straight to a v_accvgpr_read of its last
register, with no wait states on that edge.  See tests/mfma_hazards.py for
the rule checked here.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mfma_hazards import scan
from stream_residual_mixing_amd import build as B

# the shape of the case above, as the compiler emitted it
SNIPPET = """\
_Zkernel:
\tv_mfma_f32_16x16x32_bf16 a[28:31], v[132:135], v[34:37], a[28:31]
\ts_waitcnt lgkmcnt(0)
\tv_mfma_f32_16x16x32_bf16 a[28:31], v[136:139], v[34:37], a[28:31]
\ts_cbranch_vccnz .LBB0_2
\tds_read_b128 v[112:115], v79 offset:1024
\tv_accvgpr_write_b32 a0, v110
\ts_nop 7
\ts_nop 3
.LBB0_2:
\tv_accvgpr_read_b32 v115, a31
\ts_endpgm
"""


def test_scan_finds_a_read_through_a_branch():
    found = scan(SNIPPET)
    assert [(f[1], f[3]) for f in found] == [(11, ('.LBB0_2',)), (11, ('.LBB0_2',))]
    # with enough wait states on the taken edge there is nothing to report
    fixed = SNIPPET.replace(".LBB0_2:\n", ".LBB0_2:\n\ts_nop 7\n\ts_nop 3\n")
    assert scan(fixed) == []


@pytest.mark.timeout(600)
def test_library_kernels_have_no_early_mfma_reads(tmp_path):
    if not shutil.which("hipcc") and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")

    def asm(src):
        out = tmp_path / (os.path.splitext(src)[0] + ".s")
        cmd = [B.hipcc(), *[f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")], "-S",
               "--cuda-device-only", "-I", B.INCLUDE, "-I", B.CSRC, os.path.join(B.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, out.read_text()

    with ThreadPoolExecutor(min(8, len(B.SOURCES))) as ex:
        outs = list(ex.map(asm, B.SOURCES))
    n_mfma = sum(text.count("v_mfma_") for _, text in outs)
    assert n_mfma > 1000, f"only {n_mfma} MFMA instructions in the gfx950 assembly"
    bad = {src: scan(text)[:5] for src, text in outs if scan(text)}
    assert not bad, bad
    # and no kernel spills registers to scratch memory: a spill turns a
    # register-resident tile into memory traffic the byte models do not count
    # (a bf16 conversion form once made the one-pass pre kernel spill 236
    # bytes per lane, with 1.1 GB of scratch writes per call)
    spills = {}
    for src, text in outs:
        for line in text.splitlines():
            m = re.match(r"\s*\.set\s+(\S+)\.private_seg_size,\s*(.+?)\s*$", line)
            if m and m.group(2) != "0":
                spills.setdefault(src, []).append((m.group(1)[:80], m.group(2)[:40]))
    assert not spills, spills
