"""The attention kernel writes m0 in inline asm (the LDS base of each
LDS-DMA copy) and does not restore it.  That is only sound while nothing the
compiler emits in that file reads m0.  This builds the file's gfx950 device
assembly and checks it: every m0 operand is the destination of an
s_mov_b32, every LDS-DMA copy directly follows such a write (the asm helpers'
pattern), and no instruction that reads m0 implicitly is present.
"""
import os
import re
import subprocess

import pytest

from compressed_kv_cache_mla_amd import build as B

SOURCES = ["decode_mfma.hip", "sparse.hip"]

# instructions that read m0 without naming it
IMPLICIT_M0 = re.compile(r"^\s*(s_sendmsg|s_movrel|v_movrel|s_set_gpr_idx|ds_gws|ds_append|ds_consume|"
                         r"ds_ordered_count|v_interp|buffer_load_\w+.*\blds\b|buffer_store_lds)")
LDS_DMA = re.compile(r"^\s*global_load_lds_dword")
M0_WRITE = re.compile(r"^\s*s_mov_b32\s+m0,\s*s\d+\s*$")


def _device_asm(src, out):
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", "-o", out, os.path.join(B.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return [l.split(";")[0].rstrip() for l in open(out)]


@pytest.mark.parametrize("src", SOURCES)
def test_m0_written_only_by_the_copy_helpers(src, tmp_path):
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not installed")
    lines = [l for l in _device_asm(src, str(tmp_path / "k.s")) if l.strip() and not l.lstrip().startswith(".")]
    n_dma = 0
    for i, l in enumerate(lines):
        if re.search(r"\bm0\b", l):
            assert M0_WRITE.match(l), f"{src}: m0 used outside the copy helpers: {l.strip()}"
        assert not IMPLICIT_M0.match(l), f"{src}: instruction reading m0 implicitly: {l.strip()}"
        if LDS_DMA.match(l):
            n_dma += 1
            assert lines[i - 1].strip() == "s_nop 0" and M0_WRITE.match(lines[i - 2]), \
                f"{src}: LDS-DMA copy not issued by a helper: {l.strip()}"
    assert n_dma > 0
