"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libskv_host_asan.so (runtime + null device backend, g++
-fsanitize=address,undefined, every report fatal) and runs the host-library
tests against it in a child process with the sanitizer runtimes preloaded:
the hand-worked page-table fixture, the random op sequences against the
oracle's store model, and every plan limit. Any sanitizer report fails the run.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from lora_shared_kv_amd import skv
skv.library_path = lambda kind="gpu": {lib!r} if kind == "host" else skv._PKG + "/libskv.so"
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                      {tests!r} + "/test_layout_lib.py", {tests!r} + "/test_plan_limits.py"]))
"""


def test_host_runtime_under_sanitizers():
    from lora_shared_kv_amd.build import build_asan
    lib = build_asan(verbose=False)
    gcc = lambda name: subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                                      text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=gcc("libasan.so") + ":" + gcc("libubsan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
