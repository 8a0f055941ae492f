"""Host-side checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU).

The library's sources are compiled with the sanitizers on the host code only
(``-Xarch_host -fsanitize=...``; the gfx950 device code is built as usual)
and linked into ``tests/host_checks.cpp``, which drives every entry point
through argument validation and workspace sizing.  A sanitizer finding
(out-of-bounds access, overflow, misaligned access, use after free) aborts
the program with a nonzero status.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from dense_decoder_only_rmsnorm_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = B.HIPCC
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    flags = [f for f in B.FLAGS if f != "-fPIC"] + ["-O1", "-g"] + SAN

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj], capture_output=True,
                           text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    exe = str(tmp_path / "host_checks")
    drv = str(tmp_path / "host_checks.o")
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang++"
    r = subprocess.run([clang, f"-I{B.INCLUDE}", "-O1", "-g", "-fsanitize=address", "-fsanitize=undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-c",
                        os.path.join(HERE, "host_checks.cpp"), "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # linked by the host compiler with the HIP runtime: the objects already hold
    # their gfx950 code, and no hipcc line carries a sanitizer flag
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    r = subprocess.run([clang, "-fsanitize=address", "-fsanitize=undefined", drv, *objs, f"-L{rocm}/lib",
                        f"-Wl,-rpath,{rocm}/lib", "-lamdhip64", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # leaks inside the HIP runtime's own initialisation are not the library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = env.get("HIP_VISIBLE_DEVICES", "")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"stdout:\n{r.stdout}\nstderr:\n{r.stderr[-5000:]}"
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
