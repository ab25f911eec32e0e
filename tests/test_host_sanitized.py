"""The round engine's host bookkeeping (csrc/ssb_host.h: configuration check, KV page allocator,
rewind, accept record, transactional batch commit, error conversion) built as a plain CPU program
with AddressSanitizer and UndefinedBehaviorSanitizer and run; the engine library compiles the same
header, so these are the code paths its ABI calls take on the host.

A control build hands the page allocator a table one entry short and must be stopped by
AddressSanitizer, which shows the instrumentation is live."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "self_speculative_block_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "ssb_host_check.cpp")
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-static-libasan"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build(tmp_path, name, extra=()):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / name)
    subprocess.run([gxx, *FLAGS, *extra, "-I", CSRC, SRC, "-o", exe], check=True, timeout=300)
    return exe


def test_host_bookkeeping_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path, "ssb_host_check")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr


def test_sanitizer_control_catches_a_short_page_table(tmp_path):
    exe = _build(tmp_path, "ssb_host_control", ["-DSSB_HOST_CHECK_CONTROL"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
    assert "PageList::ensure" in r.stderr
