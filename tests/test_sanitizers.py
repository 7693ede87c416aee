"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code, CPU only.

* The oracle, built with gcc and -fsanitize=address,undefined, runs its pins
  in a child process with the sanitizer runtime preloaded (the interpreter
  itself is not instrumented).
* The library's host code (argument validation, the C-ABI entry points up
  to their first HIP call, status strings) is built with the sanitizers on
  the host side only: hipcc applies each -fsanitize that follows -Xarch_host
  to the host compilation, never to device code.  The CPU ABI tests then run
  against that build in a child process (SERAC_LIBRARY_PATH selects it).

Any report aborts the child (halt_on_error, no recovery from UB), and the
test fails with its output.
"""
import glob
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
SRC = os.path.join(ROOT, "sift_descriptor_nearest_amd", "csrc", "serac.hip")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")

ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def child(cmd, preload, extra_env=None, timeout=600):
    env = dict(os.environ)
    env.update(ENV)
    env.update(extra_env or {})
    env["LD_PRELOAD"] = preload
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=timeout,
                       cwd=ROOT)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    return out


def gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    oracle.build(extra=("-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", "-g"), out=lib)
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {TESTS!r})\n"
            "import oracle\n"
            "from oracle_pins import PINS\n"
            f"L = oracle.load({lib!r})\n"
            "for pin in PINS:\n"
            "    pin(L)\n"
            "    print('ok', pin.__name__, flush=True)\n")
    out = child([sys.executable, "-c", code], gcc_runtime("libasan.so"),
                {"OMP_NUM_THREADS": "4"})
    assert out.count("ok ") == 9


def test_library_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("no hipcc")
    rts = glob.glob(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "lib",
                                 "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("no clang ASan runtime")
    lib = str(tmp_path / "libserac_san.so")
    # device code as usual (at -O1: only the host side is exercised here);
    # every -fsanitize is preceded by -Xarch_host
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", INCLUDE, SRC, "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    out = child([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                 os.path.join(TESTS, "test_abi_cpu.py")], rts[0],
                {"SERAC_LIBRARY_PATH": lib})
    assert " passed" in out and "failed" not in out, out
