"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the fp64
oracle (every pin of the forward recurrence and of its reverse mode) and the C-ABI validation
layer (every bad-argument and launch-limit check of test_abi_cpu.py, with the kernel launchers
replaced by no-op test doubles from sanitizer_stubs.cpp).  Each runs in a child Python process
with the sanitizer runtime preloaded; any report fails the test."""
import os
import subprocess
import sys

import pytest

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not path or not os.path.exists(path):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    return path


def _run_child(code_or_args, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = _asan_runtime()
    # Python itself leaks by design at exit; the checks here are for memory errors and UB
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, TESTS, env.get("PYTHONPATH", "")])
    res = subprocess.run([sys.executable, *code_or_args], capture_output=True, text=True, env=env, cwd=ROOT,
                         timeout=600)
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = oracle.build(oracle.SOURCE, str(tmp_path / "oracle_san.so"), extra_flags=tuple(SAN))
    code = (
        "import oracle, oracle_pins, backward_pins\n"
        f"orc = oracle.Oracle({lib!r})\n"
        "for pin in oracle_pins.ALL_PINS + backward_pins.ALL_PINS:\n"
        "    pin(orc)\n"
        "print('pins ok', len(oracle_pins.ALL_PINS) + len(backward_pins.ALL_PINS))\n")
    out = _run_child(["-c", code], {})
    assert "pins ok" in out


def test_abi_validation_under_sanitizers(tmp_path):
    lib = str(tmp_path / "kda_abi_san.so")
    csrc = os.path.join(ROOT, "gated_delta_rule_51_amd", "csrc")
    # the host validation layer is plain C++: built by g++ (no device code), with the stubs
    cmd = ["g++", "-std=c++17", "-shared", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, "-x", "c++", os.path.join(csrc, "api.cpp"),
           os.path.join(TESTS, "sanitizer_stubs.cpp"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "hip" in res.stderr and "No such file" in res.stderr:
        pytest.skip("ROCm headers not found")
    assert res.returncode == 0, res.stderr[-3000:]
    out = _run_child(["-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(TESTS, "test_abi_cpu.py"),
                      "-k", "reject or limits or arguments or noalloc or workspace_bytes or status"],
                     {"KDA_ABI_TEST_LIBRARY": lib})
    assert " passed" in out and " failed" not in out, out[-3000:]
