"""The prefill tile reads its V operands from LDS in inline assembly, which the
compiler's wait insertion does not see: every use must follow an
`s_waitcnt lgkmcnt(0)`.  Checked on the AMD assembly of attend.hip as the
build compiles it (CPU only: hipcc cross-compiles for gfx950)."""
import os
import shutil
import subprocess
import tempfile

import pytest

from tests.asm_lds_check import asm_lds_reads, violations

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_varlen_amd", "csrc")


def test_checker_flags_an_early_use():
    # a use of a pending destination between the read and the wait is flagged;
    # the same code with the wait first is not
    asm = """_Zkernel:
\t;;#ASMSTART
\tds_read_b128 v[8:11], v2 offset:0
\t;;#ASMEND
\tv_mov_b32_e32 v20, v9
\ts_waitcnt lgkmcnt(0)
\tv_mov_b32_e32 v21, v10
"""
    bad = violations(asm)
    assert len(bad) == 1 and "v_mov_b32_e32 v20, v9" in bad[0][2]
    good = asm.replace("\tv_mov_b32_e32 v20, v9\n\ts_waitcnt lgkmcnt(0)\n",
                       "\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32_e32 v20, v9\n")
    assert violations(good) == []
    # a read-pair destination and a scratch store of it
    asm2 = """_Zk2:
\t;;#ASMSTART
\tds_read2st64_b64 v[4:7], v1 offset0:0 offset1:8
\t;;#ASMEND
\tscratch_store_dwordx4 off, v[4:7], off
"""
    assert len(violations(asm2)) == 1
    # a combined wait clears it; an unrelated register is not flagged
    asm3 = asm2.replace("\tscratch_store_dwordx4 off, v[4:7], off\n",
                        "\tv_add_u32_e32 v30, v31, v32\n\ts_waitcnt vmcnt(0) lgkmcnt(0)\n"
                        "\tscratch_store_dwordx4 off, v[4:7], off\n")
    assert violations(asm3) == []


def test_attend_asm_lds_reads_are_waited_for():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    import paged_kv_cache_varlen_amd._build as b
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "attend.s")
        cmd = [hipcc] + b.COMMON + b.EXTRA.get("attend.hip", []) + [
            "--cuda-device-only", "-S", os.path.join(CSRC, "attend.hip"), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    assert asm_lds_reads(text) > 0          # the check sees the reads it is about
    bad = violations(text)
    assert bad == [], bad[:10]
