"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  The four sources are compiled for the host only, each sanitizer
flag given to the host compilation alone (-Xarch_host), and linked with
tests/host_asan/driver.cpp, which drives the config validation, the packed,
state and workspace layout planning and the host-side argument checks of every
entry point on known shapes and 20,000 fuzzed configs (nothing reaches the
GPU).  Any out-of-bounds access, leak, use after free, signed overflow or other
undefined behaviour fails the run."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from vocoder_rvq_codebook_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")
HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not HIPCC, reason="hipcc not available")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN
    cmds, objs = [], []
    for src in B.SOURCES + ["driver.cpp"]:
        path = os.path.join(HERE, "host_asan", src) if src == "driver.cpp" else os.path.join(B.CSRC, src)
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmds.append([HIPCC, *flags, "-c", path, "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(_run, cmds))
    exe = str(tmp_path / "driver")
    _run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert "host checks passed" in r.stdout, r.stdout + r.stderr
