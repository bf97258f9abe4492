"""The host side of libmla.so under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The library is rebuilt from the same sources with the host code instrumented
(each -fsanitize= is given to the host compilation only; the gfx950 device
code is built as usual and never runs here), and tests/sanitize/abi_misuse.c
drives every entry point with one bad or extreme argument at a time: null and
misaligned pointers, sizes at 0, at the limits and at the integer extremes,
small workspaces, and the largest shapes the checks accept (which reach the
HIP launch and fail there for want of a device).  A sanitizer report, or any
status other than the expected one, fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from compressed_kv_cache_mla_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_misuse.c")
CLANG = "/opt/rocm/llvm/bin/clang"
ROCM_LIB = "/opt/rocm/lib"

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tools_present():
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return os.path.exists(CLANG) and os.path.isdir(ROCM_LIB)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{msgs}"


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    if not _tools_present():
        pytest.skip("hipcc / ROCm clang not installed")
    out = tmp_path_factory.mktemp("san")
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-O3", "-shared")] + ["-O1", "-g"] + SAN_HOST
    srcs = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))
    objs = [str(out / (s[:-4] + ".o")) for s in srcs]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: _run([B.hipcc(), *flags, "-c", "-o", so[1], os.path.join(B.CSRC, so[0])]),
                    zip(srcs, objs)))
    lib = str(out / "libmla_san.so")
    _run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *SAN_HOST, "-o", lib, *objs])
    exe = str(out / "abi_misuse")
    _run([CLANG, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-o", exe,
          DRIVER, lib, f"-Wl,-rpath,{out}", f"-L{ROCM_LIB}", "-lamdhip64", f"-Wl,-rpath,{ROCM_LIB}"])
    yield exe
    shutil.rmtree(out, ignore_errors=True)


@pytest.mark.timeout(600)
def test_abi_misuse_under_asan_ubsan(sanitized_driver):
    env = dict(os.environ)
    # leaks: the HIP runtime keeps allocations for the process lifetime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    last = [l for l in out.splitlines() if l.endswith("failed")]
    assert last and last[-1].endswith(" 0 failed"), out[-4000:]
    assert int(last[-1].split()[0]) >= 500
