"""Host code and the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled with the sanitizers on their host side
only (the device code is the same gfx950 code as the product's) and linked
into tests/sanitize/abi_check.cpp, which drives the C ABI's validation paths,
workspace sizing and schedule rule (no call reaches a HIP launch, so no GPU
is needed). The oracle is compiled with gcc and both sanitizers and run by
tests/sanitize/oracle_check.c over a small layer in every mode. A sanitizer
report aborts the program, which fails the test."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1",
           OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not found")
def test_abi_host_code_under_sanitizers(tmp_path):
    srcs = sorted(os.path.join(ROOT, "blocked_prefill_amd", "csrc", f)
                  for f in os.listdir(os.path.join(ROOT, "blocked_prefill_amd", "csrc")) if f.endswith(".hip"))
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops"]
    with ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        list(ex.map(lambda so: _run([HIPCC, *common, *HOST_SAN, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    drv = str(tmp_path / "abi_check.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(SAN, "abi_check.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_check")
    _run([CLANGXX, "-fsanitize=address,undefined", *objs, drv, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    out = _run([exe], env=ENV)
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fopenmp", os.path.join(ROOT, "oracle", "rt_oracle.c"),
          os.path.join(SAN, "oracle_check.c"), "-lm", "-o", exe])
    out = _run([exe], env=ENV)
    assert "ok" in out
