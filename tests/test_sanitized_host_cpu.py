"""The C ABI's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/abi_errors.c calls every entry point with
arguments the library must reject or answer before any kernel is enqueued
(bad layouts, NULL buffers, negative and int32/int64-limit sizes, a grid of
workspace queries up to the argument block's limits, the allocation-free
entry point's scratch limit).  It runs against a copy of the library whose
host code is built with both sanitizers (the build step makes it); any
sanitizer report or wrong return code fails it.  No GPU is used."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_errors_san")


def test_abi_error_paths_under_address_and_undefined_behavior_sanitizers():
    assert os.path.exists(DRIVER), "tests/abi_errors_san is missing: run the build step (__graft_entry__.build())"
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([DRIVER], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
