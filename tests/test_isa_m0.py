"""The LDS copies (global_load_lds) set M0 inside their own inline asm.  The
compiler is not told about that register beyond a clobber, so these kernels are
only safe while no instruction the compiler generates reads or writes M0 (for
example dynamic register indexing).  Compile each source that issues such
copies to gfx950 assembly and check that M0 appears only inside inline asm
blocks.  Host-only: hipcc cross-compiles, nothing runs on a GPU."""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from speculative_verify_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["verify.hip", "prefill.hip", "attn.hip"]


def m0_outside_asm(asm_text):
    inside, hits = False, []
    for line in asm_text.splitlines():
        if ";;#ASMSTART" in line:
            inside = True
            continue
        if ";;#ASMEND" in line:
            inside = False
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")):
            continue
        if not inside and (re.search(r"\bm0\b", t) or "movrel" in t or "gpr_idx" in t):
            hits.append(t)
    return hits


def compile_to_asm(src, out_dir):
    out = os.path.join(out_dir, src.replace(".hip", ".s"))
    cmd = [build._hipcc(), *build.HIPFLAGS, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return src, f.read()


def test_m0_is_only_touched_by_the_copies(tmp_path):
    try:
        build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: compile_to_asm(s, str(tmp_path)), SOURCES))
    for src, text in results:
        assert ";;#ASMSTART" in text, src   # the copies are there
        hits = m0_outside_asm(text)
        assert not hits, (src, hits[:5])


def test_the_check_sees_a_compiler_m0_use():
    """The scan itself: an M0 write outside an asm block is reported, one inside
    is not."""
    text = "\n".join(["\ts_mov_b32 m0, s4", "\t;;#ASMSTART", "\ts_mov_b32 m0, s5",
                      "\tglobal_load_lds_dwordx4 v[0:1], off", "\t;;#ASMEND", "\tv_movrels_b32 v0, v1"])
    assert m0_outside_asm(text) == ["s_mov_b32 m0, s4", "v_movrels_b32 v0, v1"]
