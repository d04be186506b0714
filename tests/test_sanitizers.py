"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the C oracle and its all-cores harness, every entry point driven on small
  inputs and edge cases (tests/sanitize/oracle_driver.c), leak checking on;
* a plain C99 client of libqad (tests/sanitize/client_driver.c) that drives
  the host-side validation of every entry point, built with the sanitizers
  against the normal library, and against a build of the library whose host
  code is itself sanitized (device code is not: GPU sanitizers are not used
  here).  No call of the client reaches the GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g"]


def _run(exe, env_extra=None, timeout=120):
    env = dict(os.environ)
    env.update(env_extra or {})
    out = subprocess.run([exe], capture_output=True, text=True, timeout=timeout, env=env)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), (out.returncode, out.stdout[-2000:],
                                                                         out.stderr[-4000:])


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-std=c11", "-O1", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-Wall"] + SAN_FLAGS
                   + ["-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "oracle.c"),
                      os.path.join(ROOT, "oracle", "oracle_omp.c"), os.path.join(SAN, "oracle_driver.c"), "-lm",
                      "-o", exe], check=True)
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "4"})


def _client(tmp_path, libdir, name, cc="gcc"):
    exe = str(tmp_path / name)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic"] + SAN_FLAGS
                   + ["-I", os.path.join(ROOT, "include"), os.path.join(SAN, "client_driver.c"), "-o", exe,
                      "-L", libdir, "-lqad", "-Wl,-rpath," + libdir], check=True)
    return exe


def test_c_client_under_sanitizers(tmp_path):
    from nvfp4_quantization_aware_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqad.so not built")
    # the HIP runtime keeps process-lifetime allocations: leaks are not checked
    _run(_client(tmp_path, os.path.dirname(_lib.LIB_PATH), "client"), {"ASAN_OPTIONS": "detect_leaks=0"})


def test_library_host_code_under_sanitizers(tmp_path):
    from nvfp4_quantization_aware_amd import build
    libdir = tmp_path / "lib"
    libdir.mkdir()
    # the host half of every source instrumented; each -fsanitize applies to
    # the host compilation only (-Xarch_host directly before it)
    flags = [f for f in build.compile_flags() if f not in ("-O3",)] + ["-O1", "-g", "-Xarch_host",
                                                                       "-fsanitize=address", "-Xarch_host",
                                                                       "-fsanitize=undefined"]
    objs, procs = [], []
    for src in build.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([build.hipcc()] + flags + ["-c", os.path.join(build.CSRC, src), "-o", obj],
                                      stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-3000:]
    lib = str(libdir / "libqad.so")
    subprocess.run([build.hipcc(), "--offload-arch=" + build.ARCH, "-shared", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-o", lib] + objs + build.LIBS, check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    # the library's host code carries the ROCm clang sanitizer runtime: the
    # client is built by the same clang so that one runtime serves both
    clang = os.path.join(os.path.dirname(build.hipcc()), "..", "lib", "llvm", "bin", "clang")
    _run(_client(tmp_path, str(libdir), "client_san_lib", cc=clang), {"ASAN_OPTIONS": "detect_leaks=0"})
