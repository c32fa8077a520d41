"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/attention_oracle.c) built with gcc
  -fsanitize=address,undefined runs its pins (tests/test_oracle_pins.py,
  tests/test_oracle_grads.py) in a child process with gcc's sanitizer runtimes
  preloaded.
* The library's host runtime (every source of libra.so, sanitizers on the host
  side only: device code cannot be instrumented) runs the C-ABI host tests
  (tests/test_abi_host.py) with clang's ASan runtime preloaded.
* A planted heap overflow in a throwaway C file must be reported by the same
  set-up, so a clean run means something.

Both child processes stop at the first sanitizer report (halt_on_error); leak
checking is off because the Python interpreter itself keeps allocations alive
at exit.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_attention_step_amd", "csrc")
SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtimes():
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"gcc's {name} is not installed")
        out.append(p)
    return out


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        pytest.skip("clang's ASan runtime is not installed")
    return found[-1]


def _pytest_child(env_extra, args):
    env = dict(os.environ)
    env.update(SAN_OPTS)
    env.update(env_extra)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *args],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)


def _clean(r):
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert "ERROR: AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]


def test_sanitizer_setup_reports_a_planted_overflow(tmp_path):
    asan, ubsan = _gcc_runtimes()
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int read_past_end(int n) { int* a = malloc(n * sizeof(int)); for (int i = 0; i < n; ++i) a[i] = i;\n"
                   "  int s = a[n]; free(a); return s; }\n")
    so = tmp_path / "liboverflow.so"
    subprocess.run(["gcc", "-O0", "-g", "-fsanitize=address,undefined", "-shared", "-fPIC", str(src), "-o", str(so)],
                   check=True)
    env = dict(os.environ)
    env.update(SAN_OPTS)
    env["LD_PRELOAD"] = f"{asan} {ubsan}"
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({str(so)!r}).read_past_end(7)"],
                       env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtimes()
    so = tmp_path / "libra_oracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    os.path.join(ROOT, "oracle", "attention_oracle.c"), "-o", str(so), "-lm"], check=True)
    r = _pytest_child({"LD_PRELOAD": f"{asan} {ubsan}", "RA_ORACLE_LIBRARY": str(so)},
                      ["tests/test_oracle_pins.py", "tests/test_oracle_grads.py"])
    _clean(r)


def test_host_runtime_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not installed")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [hipcc, "-O1", "-g", "-std=c++20", "-fPIC", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
               "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    so = str(tmp_path / "libra_san.so")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", so],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = _pytest_child({"LD_PRELOAD": rt, "RA_LIBRARY": so}, ["tests/test_abi_host.py"])
    _clean(r)
    assert " passed" in r.stdout
