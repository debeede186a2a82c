"""The host logic of libveda under AddressSanitizer and UndefinedBehavior-
Sanitizer: csrc/host.cpp and csrc/api_host.cpp are built with g++ into a
host-only library, and tests/test_lib_host.py runs against it in a child
Python with the ASan runtime preloaded. Any sanitizer report aborts the
child, so the run fails on the first memory or undefined-behaviour error."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    gxx = shutil.which("g++")
    if gxx is None:
        return None
    path = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_logic_under_sanitizers():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("g++ with the ASan runtime is not available")
    from learned_block_sparse_amd.build import build_host_sanitized
    lib = build_host_sanitized()
    env = dict(os.environ)
    env.update(
        LD_PRELOAD=asan,
        VEDA_LIBRARY=lib,
        # Python itself keeps memory until exit; leaks are not what is checked
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
        CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="",
    )
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_lib_host.py"),
                        "-k", "not attention_unsupported and not full_attention_layers"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert " passed" in r.stdout
