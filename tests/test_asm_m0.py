"""The direct global->LDS loads (dma16s / dma16v in csrc/common.h) set M0 inside inline asm
and list it as clobbered. clang warns that the clobber of a reserved register may not be
honoured, so the pattern is safe only while no compiler-generated instruction of these
kernels uses M0 (a value the compiler put there could be overwritten by the helpers).
This test compiles the sources that use the helpers to gfx950 assembly with the library's
own flags and checks that every M0 reference is one of the helpers' two instructions."""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from diffusion_transformer_mmdit_amd import build as B

SOURCES = ("gemm.hip", "attention.hip")
OWN = (re.compile(r"^\s*s_mov_b32 m0, s\d+\s*$"), re.compile(r"^\s*global_load_lds_dwordx4 "))
# instructions that read M0 without naming it in the assembly text
IMPLICIT = re.compile(r"^\s*(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_append|ds_consume|"
                      r"ds_ordered_count|\w*_addtid|v_interp|buffer_load_lds|s_ttracedata)")


def _asm(src, tmp):
    out = os.path.join(tmp, src + ".s")
    cmd = [B.hipcc(), "-x", "hip"] + B.common_flags() + [
        "-S", "--cuda-device-only", os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-2000:]}"
    with open(out) as f:
        return f.read()


@pytest.mark.slow
def test_m0_is_used_only_by_the_direct_load_helpers():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _asm(s, tmp), SOURCES))
    for src, text in zip(SOURCES, texts):
        # instruction lines only (comments and directives may name m0 too)
        lines = [ln.split(";")[0] for ln in text.splitlines()]
        refs = [ln for ln in lines if re.search(r"\bm0\b", ln)]
        writes = [ln for ln in refs if OWN[0].match(ln)]
        assert writes, f"{src}: the direct-load helpers are no longer used"
        other = [ln.strip() for ln in refs if not any(p.match(ln) for p in OWN)]
        assert not other, f"{src}: compiler-generated M0 uses: {sorted(set(other))[:5]}"
        implicit = sorted({ln.split()[0] for ln in lines if IMPLICIT.match(ln)})
        assert not implicit, f"{src}: instructions with an implicit M0 operand: {implicit}"
        # every direct load follows its own M0 write
        loads = [ln for ln in lines if OWN[1].match(ln)]
        assert len(loads) == len(writes), f"{src}: {len(loads)} direct loads, {len(writes)} M0 writes"
