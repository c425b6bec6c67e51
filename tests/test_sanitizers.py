"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Three drivers under tests/sanitize/ are built with the sanitizers on the
host side and run:

- bm_driver: random operation sequences through the C++ block manager
  (pa_block_manager.hip is host-only C++; it is compiled from a .cpp copy),
  checking the bookkeeping against token read-back through the tables;
- api_driver: the C ABI's argument checks, workspace sizes and path queries
  (pa_api.hip built with host-side sanitizers and linked with the library's
  other objects); every call there is refused or answered before a launch,
  so no kernel ever sees its fake addresses;
- oracle_driver: the fp64 CPU oracle on random shapes in every storage type.

Any sanitizer report fails the run (-fno-sanitize-recover=all; leaks are
reported at exit).  Sanitized device code is never built: on the hipcc lines
each sanitizer flag sits behind -Xarch_host.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from paged_kv_cache_405_amd import build as B  # noqa: E402

SAN = os.path.join(ROOT, "tests", "sanitize")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r.stdout


def _gxx():
    for c in ("g++", "c++"):
        if shutil.which(c):
            return c
    pytest.skip("no host C++ compiler")


def test_block_manager_under_sanitizers(tmp_path):
    src = tmp_path / "pa_block_manager_host.cpp"       # host-only C++: built from a plain .cpp copy
    shutil.copy(os.path.join(ROOT, "paged_kv_cache_405_amd", "csrc", "pa_block_manager.hip"), src)
    exe = tmp_path / "bm_driver"
    _run([_gxx(), "-O1", "-g", "-std=c++17"] + GCC_SAN + [f"-I{os.path.join(ROOT, 'include')}",
         os.path.join(SAN, "bm_driver.cpp"), str(src), "-o", str(exe)])
    for seed in (1, 2, 3):
        out = _run([str(exe), str(seed), "3000"], env=ENV)
        assert "clean" in out


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("no gcc")
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off"] + GCC_SAN +
         [os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "pa_oracle.c"), "-o", str(exe), "-lm"])
    out = _run([str(exe), "5", "1500"], env=ENV)
    assert "clean" in out


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_api_checks_under_sanitizers(tmp_path):
    objdir = B.OBJDIR
    others = sorted(os.path.join(objdir, f) for f in os.listdir(objdir)
                    if f.endswith(".o") and f != "pa_api.hip.o") if os.path.isdir(objdir) else []
    if len(others) < len(B.sources()) - 1:
        B.build()                                       # the library's own objects, unsanitized
        others = sorted(os.path.join(objdir, f) for f in os.listdir(objdir)
                        if f.endswith(".o") and f != "pa_api.hip.o")
    api_o, drv_o, exe = tmp_path / "pa_api.o", tmp_path / "api_driver.o", tmp_path / "api_driver"
    _run([B.HIPCC] + [f for f in B.CFLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN +
         ["-c", os.path.join(ROOT, "paged_kv_cache_405_amd", "csrc", "pa_api.hip"), "-o", str(api_o)])
    _run([B.HIPCC, "-O1", "-g", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}"] + HOST_SAN +
         ["-c", os.path.join(SAN, "api_driver.cpp"), "-o", str(drv_o)])
    _run([B.HIPCC, f"--offload-arch={B.ARCH}"] + HOST_SAN[:4] + [str(drv_o), str(api_o)] + others +
         ["-o", str(exe)])
    out = _run([str(exe)], env=ENV)
    assert "clean" in out
