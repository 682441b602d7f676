"""The host launch tables of libzero, and the CPU oracle's C code, checked
on the CPU under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/host_tables.cpp is compiled with the library's host code
(zero_api.cpp) in place of the HIP launchers.  Its stand-in launchers replay
the kernels' workgroup-to-work indexing over the argument blocks the host
code builds.  For a few hundred random plans it checks two things:

- flatten, gather_pack and reshard write every destination element exactly
  once, and read only inside their sources;
- the Adam step and the reduction cover the owner's shard at the plan's full
  and destination offsets (the ownership rule of the ZeRO pages' partitioning
  figure), in rank groups of at most 128.

It also covers plans with more buckets than one launch's table, and a shard
longer than 2^28 elements.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_launch_tables(tmp_path):
    exe = tmp_path / "host_tables"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "zero_sharded_mixed_02_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "host_tables.cpp"),
           os.path.join(ROOT, "zero_sharded_mixed_02_amd", "csrc", "zero_api.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    """The CPU oracle's C entry points on edge inputs (zero counts, 1 and 130
    ranks, every 16-bit pattern decoded, a strided fp32 sweep encoded,
    NaN/Inf/denormal Adam inputs) under AddressSanitizer and UBSan."""
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-Wall", "-Wextra", "-Werror", os.path.join(ROOT, "tests", "native", "oracle_sanitize.c"),
           os.path.join(ROOT, "oracle", "zero_oracle.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitize ok" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_thread_safety(tmp_path):
    """libzero's host code from eight threads at once (own and shared plans,
    every entry point, per-thread error text) while another thread changes
    the write-window setting, under ThreadSanitizer."""
    exe = tmp_path / "host_threads"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "zero_sharded_mixed_02_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "host_threads.cpp"),
           os.path.join(ROOT, "zero_sharded_mixed_02_amd", "csrc", "zero_api.cpp"),
           "-o", str(exe), "-pthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
