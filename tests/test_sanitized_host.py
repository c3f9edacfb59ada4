"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each exercised by the existing CPU tests in a child process that preloads its
sanitizer runtime (an instrumented library cannot be loaded into a process whose first
library is not the runtime):
  - the C oracle, built by gcc with -fsanitize=address,undefined, under its pins;
  - the library's host side (argument checks, overlap and alignment rules, launch plans and
    workspace sizes), built by hipcc with the host pass instrumented and the device code as
    usual, under the C-ABI host tests.
A sanitizer report fails the child (halt_on_error), and so the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG_ASAN = "/opt/rocm/lib/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"

# the child checks that the runtime is live and that the instrumented library is the one
# loaded, then runs the tests
_CHILD = r"""
import ctypes, os, sys
ctypes.CDLL(None)["__asan_init"]            # raises if no ASan runtime is in the process
sys.path.insert(0, os.environ["GDN_ROOT"])
if os.environ.get("GDN_LIB"):
    from linear_attention_recurrence_chunked_amd import gdn
    assert gdn.load()._name == os.environ["GDN_LIB"], gdn.load()._name
if os.environ.get("GDN_ORACLE_LIB"):
    import oracle
    assert oracle._load()._name == os.environ["GDN_ORACLE_LIB"], oracle._load()._name
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider"] + sys.argv[1:]))
"""


def _run_child(env_extra, tests):
    env = dict(os.environ)
    env.update(env_extra)
    env["GDN_ROOT"] = ROOT
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", _CHILD] + tests, cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    return r.stdout


def test_oracle_pins_under_asan_ubsan():
    import oracle
    lib = oracle.build(force=False, sanitize=True)
    rt = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    out = _run_child({"LD_PRELOAD": rt, "GDN_ORACLE_LIB": lib},
                     ["tests/test_oracle_pins.py", "tests/test_backward_pins.py",
                      "tests/test_channel_pins.py", "tests/test_layer_step_pins.py",
                      "tests/test_qsa_pins.py"])
    assert " passed" in out


def test_host_abi_under_asan_ubsan():
    if not os.path.exists(CLANG_ASAN):
        pytest.skip("clang ASan runtime not found at " + CLANG_ASAN)
    from linear_attention_recurrence_chunked_amd import build
    lib = build.build(sanitize=True)
    out = _run_child({"LD_PRELOAD": CLANG_ASAN, "GDN_LIB": lib}, ["tests/test_abi_host.py"])
    assert " passed" in out
