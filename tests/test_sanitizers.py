"""AddressSanitizer + UndefinedBehaviorSanitizer (no recovery, leak check on)
over the host C code, on the CPU:

- the seeded generator (synth/synth.c) and the float64 oracle
  (oracle/sps_oracle.c), built with gcc and driven by
  tests/sanitize/oracle_synth_main.c over small corpora with empty rows,
  ragged chunks, signed values and planted CSR faults;
- libsps's host code (sizing arithmetic, argument and shape checks, status
  strings, the thread-local error message), built with hipcc with the
  sanitizers on the host side only, and driven by
  tests/sanitize/host_abi_main.c through the C ABI. Every call there returns
  before any device work, so no GPU is needed and GPU code is not
  instrumented.

A negative control first shows that each toolchain's sanitizer build does
report a planted heap overflow and a planted signed overflow, so a clean
run means something.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_embedding_exact_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

C_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-g", "-O1"]
# hipcc: the sanitizers go to the host compilation only
HIP_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                "-fno-omit-frame-pointer"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

PLANT_HEAP = r"""
#include <stdlib.h>
int plant_heap(int n) { int *a = (int *)malloc(n * sizeof(int)); volatile int k = n;
  a[k] = 1; int r = a[0]; free(a); return r; }
"""
PLANT_INT = r"""
int plant_int(int x) { volatile int y = x; return y + 2147483647; }
"""
PLANT_MAIN = r"""
int plant_heap(int n); int plant_int(int x);
int main(int argc, char **argv) { (void)argv; return argc > 1 ? plant_int(argc) : plant_heap(4); }
"""


def _run(cmd, cwd, env=None, timeout=300):
    return subprocess.run(cmd, cwd=cwd, env=env, stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=timeout)


def _build(cmd, cwd):
    r = _run(cmd, cwd)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout
    return r


def _need(tool):
    if not (os.path.exists(tool) or shutil.which(tool)):
        pytest.skip(tool + " not installed")


def _expect_reports(exe, cwd):
    heap = _run([exe], cwd, ENV)
    assert heap.returncode != 0 and "heap-buffer-overflow" in heap.stdout, heap.stdout
    ovf = _run([exe, "x"], cwd, ENV)
    assert ovf.returncode != 0 and "signed integer overflow" in ovf.stdout, ovf.stdout


def test_negative_control_gcc(tmp_path):
    _need("gcc")
    d = str(tmp_path)
    for name, text in (("h.c", PLANT_HEAP), ("i.c", PLANT_INT), ("m.c", PLANT_MAIN)):
        open(os.path.join(d, name), "w").write(text)
    _build(["gcc"] + C_SAN + ["h.c", "i.c", "m.c", "-o", "plant"], d)
    _expect_reports("./plant", d)


def test_negative_control_hipcc_host(tmp_path):
    _need(HIPCC)
    _need(CLANG)
    d = str(tmp_path)
    open(os.path.join(d, "plant.hip"), "w").write(
        '#include <hip/hip_runtime.h>\nextern "C" {\n' + PLANT_HEAP + PLANT_INT + "}\n")
    open(os.path.join(d, "m.c"), "w").write(PLANT_MAIN)
    _build([HIPCC] + HIP_FLAGS + HIP_HOST_SAN + ["-o", "libplant.so", "plant.hip"], d)
    _build([CLANG] + C_SAN + ["m.c", "-L.", "-lplant", "-Wl,-rpath," + d, "-o", "plant"], d)
    _expect_reports("./plant", d)


def test_oracle_and_generator_clean(tmp_path):
    _need("gcc")
    d = str(tmp_path)
    _build(["gcc", "-std=c11", "-pthread"] + C_SAN +
           [os.path.join(SAN, "oracle_synth_main.c"), os.path.join(ROOT, "oracle", "sps_oracle.c"),
            "-lm", "-o", "osan"], d)
    r = _run(["./osan"], d, ENV)
    assert r.returncode == 0 and "clean" in r.stdout, r.stdout


def test_libsps_host_code_clean(tmp_path):
    _need(HIPCC)
    _need(CLANG)
    d = str(tmp_path)
    srcs = [os.path.join(CSRC, f) for f in ("sps_prepare.hip", "sps_score.hip", "sps_bsc.hip",
                                            "sps_api.hip")]
    _build([HIPCC] + HIP_FLAGS + HIP_HOST_SAN +
           ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", "libsps_san.so"] + srcs, d)
    _build([CLANG, "-std=c11", "-pthread"] + C_SAN +
           ["-I", os.path.join(ROOT, "include"), os.path.join(SAN, "host_abi_main.c"), "-L.",
            "-lsps_san", "-Wl,-rpath," + d, "-o", "hsan"], d)
    r = _run(["./hsan"], d, ENV)
    assert r.returncode == 0 and "clean" in r.stdout, r.stdout
