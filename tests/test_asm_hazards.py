"""The hand-issued loads of the grouped-query kernels never have their
destination registers reused while in flight (static check of the device
assembly, built with the library's own flags), and the checker itself finds
such a reuse when one is planted."""
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(__file__))
import asm_hazards  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from paged_kv_cache_405_amd import build as B  # noqa: E402


def _kernel(body: str) -> str:
    return "_Z6kernelv:\n" + body + "\n.Lfunc_end0:\n"


PLANTED = _kernel("""
\t;;#ASMSTART
\tglobal_load_dwordx4 v[2:5], v[0:1], off
\t;;#ASMEND
\tv_mov_b32_e32 v3, 0
\ts_waitcnt vmcnt(0)
\ts_endpgm""")

CLEAN = _kernel("""
\t;;#ASMSTART
\tglobal_load_dwordx4 v[2:5], v[0:1], off
\t;;#ASMEND
\tglobal_load_dword v9, v[0:1], off
\ts_waitcnt vmcnt(1)
\tv_mov_b32_e32 v3, 0
\ts_waitcnt vmcnt(0)
\ts_endpgm""")

# the wait covers the asm load only when no younger load is allowed in flight
TOO_LOOSE = _kernel("""
\t;;#ASMSTART
\tglobal_load_dwordx4 v[2:5], v[0:1], off
\t;;#ASMEND
\tglobal_load_dword v9, v[0:1], off
\ts_waitcnt vmcnt(2)
\tv_mov_b32_e32 v3, 0
\ts_endpgm""")

# pending on one branch only: still a violation at the join
BRANCHY = _kernel("""
\ts_cbranch_scc1 .LBB0_2
\t;;#ASMSTART
\tglobal_load_dwordx4 v[2:5], v[0:1], off
\t;;#ASMEND
.LBB0_2:
\tv_add_u32_e32 v4, 1, v4
\ts_waitcnt vmcnt(0)
\ts_endpgm""")

LDS_READ = _kernel("""
\t;;#ASMSTART
\tds_read_b64_tr_b16 v[6:7], v1 offset:0
\t;;#ASMEND
\tv_and_b32_e32 v6, 1, v6
\ts_waitcnt lgkmcnt(0)
\ts_endpgm""")


def test_checker_finds_planted_reuse():
    assert asm_hazards.check_assembly(PLANTED)["_Z6kernelv"]
    assert asm_hazards.check_assembly(TOO_LOOSE)["_Z6kernelv"]
    assert asm_hazards.check_assembly(BRANCHY)["_Z6kernelv"]
    assert asm_hazards.check_assembly(LDS_READ)["_Z6kernelv"]


def test_checker_accepts_covered_use():
    assert asm_hazards.check_assembly(CLEAN)["_Z6kernelv"] == []


MFMA_SOURCES = [s for s in B.sources() if "mfma" in os.path.basename(s) or "prefill" in os.path.basename(s)]


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", MFMA_SOURCES, ids=os.path.basename)
def test_no_inflight_register_reuse(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.HIPCC] + B.CFLAGS + ["--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    result = asm_hazards.check_assembly(out.read_text())
    assert result, "no kernel with inline assembly found"
    bad = {k: v[:3] for k, v in result.items() if v}
    assert not bad, bad
