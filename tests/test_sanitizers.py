"""Host sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer) of
the CPU oracle and of the C ABI's argument validation, each as a separate
program built here and run as a subprocess (no GPU: nothing reaches a
launch).  The HIP sources are built with the sanitizers on the host side
only (-Xarch_host before each -fsanitize)."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer", "-ffp-contract=off", *SAN,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "hsq_oracle.c"), "-lm",
          "-o", exe])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"), timeout=300)
    assert "oracle sanitizer run ok" in r.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_abi_validation_under_asan_ubsan(tmp_path):
    from w4a4_rank_assisted_amd import build as B

    import concurrent.futures

    host_san = [f for s in SAN for f in ("-Xarch_host", s)]

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        flags = host_san if src == "api.hip" else []
        _run([B.HIPCC, *B.CFLAGS, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    drv = str(tmp_path / "abi_driver.o")
    _run([B.HIPCC, f"--offload-arch={B.ARCH}", "-std=c++17", "-g", *host_san, f"-I{B.INCLUDE}",
          "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([B.HIPCC, f"--offload-arch={B.ARCH}", *host_san, drv, *objs, "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "abi sanitizer run ok" in r.stdout
