"""CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds, each in a child process with the ASan runtime preloaded (leak
checking off: the Python interpreter itself is not instrumented), so that an
out-of-bounds access, use-after-free or undefined operation aborts the run
instead of silently corrupting a parity result:

* the C oracle (pkv_oracle.c), rebuilt with -fsanitize=address,undefined and
  selected through PKV_ORACLE_LIB, runs the oracle pins that call it
  (test_oracle_pins.py, test_codec_pins.py);
* the C-ABI layer of the library (pkv_api.cpp: argument validation,
  workspace sizing, dispatch), built host-only with g++ against stand-ins for
  the device launchers (abi_host_stubs.cpp), runs the CPU ABI tests
  (test_abi.py), which drive every entry point's error paths.
"""
import os
import subprocess
import sys

import pytest

from oracle import c_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_decode_amd", "csrc")


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not (os.path.isabs(path) and os.path.exists(path)):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _run_child(args, extra_env):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD")
    env["LD_PRELOAD"] = _asan_runtime() + (":" + pre if pre else "")   # the ASan runtime must come first
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT + (os.pathsep + env["PYTHONPATH"] if env.get("PYTHONPATH") else "")
    env.update(extra_env)
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=850)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
    return r.stdout


@pytest.mark.timeout(900)
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = c_oracle.build(force=True, sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    _run_child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                "tests/test_oracle_pins.py", "tests/test_codec_pins.py",
                "tests/test_sanitizers.py::test_child_loaded_the_sanitized_oracle"],
               {"PKV_ORACLE_LIB": lib, "PKV_EXPECT_SANITIZED_ORACLE": lib})


def test_child_loaded_the_sanitized_oracle():
    """Run inside the child above: the oracle library in use is the sanitized
    build (skipped elsewhere)."""
    want = os.environ.get("PKV_EXPECT_SANITIZED_ORACLE")
    if not want:
        pytest.skip("only meaningful in the sanitizer child process")
    assert os.path.samefile(c_oracle.lib()._name, want)


@pytest.mark.timeout(600)
def test_abi_layer_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libpkv_host_san.so")
    cmd = ["g++", *c_oracle.SAN_FLAGS, "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "pkv_api.cpp"), os.path.join(ROOT, "tests", "abi_host_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    script = ("import sys, pytest\n"
              "import paged_kv_attention_decode_amd._native as n\n"
              f"n.LIB_PATH = {lib!r}\n"
              "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi.py']))\n")
    out = _run_child(["-c", script], {})
    assert "failed" not in out
