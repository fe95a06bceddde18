"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle: oracle/oracle.c compiled with tests/sanitize_oracle_driver.c,
  which runs every oracle function on exact-size buffers over empty, single
  block and ragged shapes and every bf16 class.
- The C ABI's argument validation: the library built with both sanitizers on
  its host code (its device code compiled as usual) and linked into
  tests/sanitize_abi_driver.cpp, which makes every entry point reject bad
  arguments, dimensions up to 2^62 included, before any HIP call.

Either program exits non-zero on a sanitizer report (no recovery) or on a
failed check."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "float8_mixed_precision_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIP_SOURCES = ("api.hip", "quantize.hip", "gemm.hip", "swiglu.hip")

# sanitizer flags for the host compilers (gcc for the oracle, clang for the driver)
HOST_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
# the same for the library: hipcc applies them to the host code only
LIB_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-gpu-sanitize"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\nexit %d\n%s%s" % (" ".join(cmd), r.returncode,
                                                     r.stdout[-3000:], r.stderr[-6000:])
    return r


def _env(**kw):
    env = dict(os.environ)
    env.update(kw)
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp"] + HOST_SAN +
         [os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(TESTS, "sanitize_oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=_env(OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1"))
    assert "0 failed checks" in r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None or
                    not os.path.exists(os.path.join(ROCM, "llvm", "bin", "clang++")),
                    reason="hipcc / ROCm clang not available")
def test_abi_validation_under_sanitizers(tmp_path):
    common = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-g", "-fno-omit-frame-pointer",
              "-Xarch_host", "-O1", "-Xarch_device", "-O1",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I" + INCLUDE] + LIB_SAN
    objs = [str(tmp_path / (s + ".o")) for s in HIP_SOURCES]
    with ThreadPoolExecutor(len(HIP_SOURCES)) as ex:
        list(ex.map(lambda so: _run(["hipcc", "-c"] + common +
                                    [os.path.join(CSRC, so[0]), "-o", so[1]], timeout=900),
                    zip(HIP_SOURCES, objs)))
    lib = str(tmp_path / "libfp8_san.so")
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"] + LIB_SAN + objs + ["-o", lib])
    exe = str(tmp_path / "abi_san")
    _run([os.path.join(ROCM, "llvm", "bin", "clang++"), "-std=c++17", "-O1", "-g",
          "-fno-omit-frame-pointer"] + HOST_SAN +
         ["-I" + INCLUDE, os.path.join(TESTS, "sanitize_abi_driver.cpp"),
          lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    # the HIP runtime's own allocations outlive main(): leak checking off
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=0"), timeout=300)
    assert "0 mismatches" in r.stdout
