"""Checks on the gfx950 code the GEMM translation unit compiles to (CPU only:
hipcc cross-compiles).  The direct-to-LDS kernels issue their loads from
inline assembly that writes m0 without the compiler's knowledge, which is
sound only while the compiler itself places nothing in m0 inside those
kernels: every m0 write there must be the asm's own, right before its load.
They also keep every operand in registers (no scratch)."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from vocoder_rvq_codebook_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")


@pytest.fixture(scope="module")
def gemm_asm():
    if not HIPCC:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "conv_gemm.s")
        cmd = [HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, "conv_gemm.hip"), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _kernels(asm, tag):
    """(symbol, body lines) of every kernel whose symbol contains tag."""
    parts = re.split(r"\n(?=_Z\S*:\s*;)", asm)
    out = []
    for p in parts:
        head = p.split("\n", 1)[0]
        if tag in head:
            out.append((head.split(":")[0], [l.strip() for l in p.splitlines()]))
    return out


def test_direct_load_kernels_own_m0(gemm_asm):
    ks = _kernels(gemm_asm, "dma_kernel")
    assert len(ks) >= 8, "direct-to-LDS kernel instances not found"
    for sym, lines in ks:
        loads = 0
        for i, l in enumerate(lines):
            if l.startswith(";") or not re.search(r"\bm0\b", l):
                continue
            assert l.startswith("s_mov_b32 m0,"), f"{sym}: m0 used by the compiler: {l}"
            assert lines[i + 1].startswith("global_load_lds_dwordx4"), f"{sym}: m0 write not followed by its load"
            loads += 1
        assert loads > 0, sym


def test_direct_load_kernels_use_no_scratch(gemm_asm):
    sizes = re.findall(r"\.amdhsa_kernel (\S*dma_kernel\S*)\n(?:.*\n)*?\s*\.amdhsa_private_segment_fixed_size (\d+)",
                       gemm_asm)
    assert len(sizes) >= 8
    for sym, n in sizes:
        assert int(n) == 0, f"{sym} spills to scratch ({n} bytes per lane)"


def _vgprs(asm):
    """{kernel symbol: VGPRs + AGPRs} from the code object metadata."""
    out = {}
    for block in asm.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        v = re.search(r"\.vgpr_count:\s+(\d+)", block)
        a = re.search(r"\.agpr_count:\s+(\d+)", block)
        if name and v:
            out[name.group(1)] = int(v.group(1)) + (int(a.group(1)) if a else 0)
    return out


def test_hot_gemm_tiles_keep_four_waves_per_simd(gemm_asm):
    """The big GEMM tiles run 8 waves per block and two blocks per CU, which
    needs at most 128 registers per lane.  Measured exceptions: the split
    (fp32-accurate) 128x128 tile needs about 150 and runs one block per CU."""
    regs = _vgprs(gemm_asm)
    hot = {k: v for k, v in regs.items()
           if re.search(r"TileCfgD?ILi(96|128)ELi128E", k) and ("conv_gemm_kernel" in k or "dma_kernel" in k)}
    assert len(hot) >= 16, sorted(regs)
    for k, v in hot.items():
        # <split-K = false, fp16 rows = false, split fp16 = true[, windows = false]>
        split_128 = "dma_kernel" in k and "ILi128ELi128E" in k and re.search(r"ELb0ELb0ELb1E(?:Lb0E)?EEv10ConvParams$", k)
        if split_128:
            continue
        assert v <= 128, f"{k}: {v} registers per lane (more than 128 halves the blocks per CU)"
