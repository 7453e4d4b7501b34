"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two drivers under tests/asan/ are built with the sanitizers and run:

  oracle_driver.c   the oracle's C reference (oracle/gemm_ref.c) on random
                    small shapes with every operand allocated to its exact
                    extent, results checked against a plain loop;
  capi_driver.cpp   the C ABI's host code (capi.cpp, sanitizers on its host
                    part only; the device code is built as usual) on random
                    and mangled layout text, the kernel-map exports at their
                    reported sizes, and the GEMM and chain argument checks
                    with dimensions up to the int64 range.  Nothing is
                    launched.

A sanitizer report makes the driver exit non-zero (-fno-sanitize-recover).
CPU only; skipped where a compiler or the library's objects are missing."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "asan")
OBJDIR = os.path.join(ROOT, "_build")
CSRC = os.path.join(ROOT, "mma_fragment_layouts_tn_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = "-fsanitize=address,undefined -fno-sanitize-recover=all".split()
# sanitizers for the host pass of a HIP compile only
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")
SEEDS = ("1", "2", "3")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return tmp_path_factory.mktemp("asan")


def test_oracle_reference_under_sanitizers(outdir):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(outdir / "oracle_driver")
    _run(["gcc", "-g", "-O1", *SAN, os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    for seed in SEEDS:
        r = _run([exe, seed], env=ENV, timeout=300)
        assert "0 mismatches" in r.stdout, r.stdout


def test_c_abi_host_code_under_sanitizers(outdir):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not available")
    objs = sorted(os.path.join(OBJDIR, f) for f in os.listdir(OBJDIR) if f.endswith(".hip.o")) \
        if os.path.isdir(OBJDIR) else []
    if not objs:
        pytest.skip("library objects not built (mma_fragment_layouts_tn_amd/_build.py)")
    capi_o, drv_o, exe = (str(outdir / n) for n in ("capi.o", "driver.o", "capi_driver"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
    _run([HIPCC, *flags, *HOST_SAN, "-Xarch_host", "-fno-sanitize-recover=all", "-c",
          os.path.join(CSRC, "capi.cpp"), "-o", capi_o])
    _run([CLANGXX, "-g", "-O1", "-std=c++17", *SAN, "-c", os.path.join(HERE, "capi_driver.cpp"),
          "-o", drv_o])
    _run([CLANGXX, *SAN[:1], drv_o, capi_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    for seed in SEEDS:
        r = _run([exe, seed], env=ENV, timeout=300)
        assert "0 failures" in r.stdout, r.stdout
