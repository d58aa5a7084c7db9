"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, no GPU call):

- the library's C ABI argument paths: every source of the library is built
  again with its host half instrumented (device half unoptimised: never
  run here) and linked into tests/sanitize/host_args.cpp, which calls every
  entry point with arguments the host answers (rejected, nothing to do, or a
  host-only query);
- the C oracle: tests/sanitize/oracle_args.c runs every oracle function on
  exactly sized arrays, against a dense brute force, plus its bad-argument
  returns.

A sanitizer report (heap overflow, leak, signed overflow, misaligned load,
...) or a failed check makes the program exit non-zero."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_dense_linear_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"

# host-side instrumentation only: each -fsanitize= goes with -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_library_host_paths_under_sanitizers(tmp_path):
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") and f != "ceiling.hip")
    flags = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-O1", "-Xarch_device", "-O0",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + HOST_SAN

    def compile_one(src):
        obj = str(tmp_path / (src[:-4] + ".o"))
        _run([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources))
    main = str(tmp_path / "host_args.o")
    _run([HIPCC, "-std=c++17", "-O1", "-Wall", "-I", os.path.join(ROOT, "include")] +
         HOST_SAN + ["-c", os.path.join(HERE, "host_args.cpp"), "-o", main])
    exe = str(tmp_path / "host_args")
    _run([HIPCC, "--offload-arch=gfx950"] + HOST_SAN + objs + [main, "-o", exe])
    r = _run([exe], env=ENV)
    assert "host argument paths: ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_args")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-Wall", "-Wextra",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(HERE, "oracle_args.c"),
          os.path.join(ROOT, "oracle", "spmm_ref.c"),
          os.path.join(ROOT, "oracle", "sddmm_ref.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle argument paths: ok" in r.stdout
