"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* The oracle is rebuilt with gcc's -fsanitize=address,undefined and its pins
  (tests/test_oracle_pins.py) run against that build in a child process that
  preloads gcc's runtimes.
* The library is rebuilt with the sanitizers on its host code (validation,
  workspace layout, FIFO bookkeeping, launch set-up; the kernels are unchanged)
  and the C-ABI tests (tests/test_abi.py) run against it in a child process
  that preloads clang's ASan runtime.
Any report aborts the child (no recovery), which fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run_child(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    lib = ob.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = {"LD_PRELOAD": f"{asan}:{ubsan}", "XL_ORACLE_LIB": lib}
    # the child really runs the sanitized build with the runtime loaded
    probe = ("import oracle, sys; oracle._load(); maps = open('/proc/self/maps').read(); "
             "assert 'libasan' in maps and oracle._LIB_PATH in maps, 'sanitized oracle not loaded'")
    _run_child(env, ["-c", probe])
    out = _run_child(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"])
    assert " passed" in out


def test_abi_under_host_asan_ubsan(tmp_path):
    rts = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang ASan runtime not installed")
    sys.path.insert(0, ROOT)
    from transformer_xl_relative_amd import build as lb
    lib = lb.build(out=str(tmp_path / "libxlrel.so"), host_sanitize=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "host code not instrumented"
    env = {"LD_PRELOAD": rts[-1], "XL_LIB": lib}
    probe = ("import transformer_xl_relative_amd as xl; xl.lib(); maps = open('/proc/self/maps').read(); "
             "assert 'libclang_rt.asan' in maps and xl.LIB_PATH in maps, 'sanitized library not loaded'")
    _run_child(env, ["-c", probe])
    out = _run_child(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"])
    assert " passed" in out
