"""Host C++ of the library under the compiler's sanitizers, on the CPU: the pool index
(csrc/pool.cpp) in a randomised model check built with AddressSanitizer +
UndefinedBehaviorSanitizer and a threaded stress of one handle built with ThreadSanitizer
(tests/pool_sanitize_driver.cpp); the shared-document planner (csrc/share.cpp) on random
batches (tests/share_sanitize_driver.cpp) and the ABI's host helpers (csrc/host.cpp: word
encoder, Llama 3.1 table, status strings; tests/host_sanitize_driver.cpp) under
AddressSanitizer + UndefinedBehaviorSanitizer. All are plain C++ with no device code, so g++
builds them on their own."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(HERE, "pool_sanitize_driver.cpp"),
       os.path.join(ROOT, "position_agnostic_kv_paged_amd", "csrc", "pool.cpp")]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


HOST_SRC = [os.path.join(HERE, "host_sanitize_driver.cpp"),
            os.path.join(ROOT, "position_agnostic_kv_paged_amd", "csrc", "host.cpp")]
SHARE_SRC = [os.path.join(HERE, "share_sanitize_driver.cpp"),
             os.path.join(ROOT, "position_agnostic_kv_paged_amd", "csrc", "share.cpp")]


def _build_and_run(tmp_path, flags, arg, env_extra, src=SRC):
    exe = str(tmp_path / "driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *flags,
           "-I", os.path.join(ROOT, "include"), *src, "-o", exe, "-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"sanitizer build unavailable: {r.stderr[-400:]}")
    env = dict(os.environ, **env_extra)
    env.pop("LD_PRELOAD", None)                  # the sanitizer runtime must load first
    r = subprocess.run([exe, arg], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])


def test_pool_index_model_check_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                   "model", {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                             "UBSAN_OPTIONS": "print_stacktrace=1"})


def test_pool_index_threaded_stress_tsan(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=thread"], "threads",
                   {"TSAN_OPTIONS": "halt_on_error=1"})


def test_share_planner_random_batches_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                   "400", {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                           "UBSAN_OPTIONS": "print_stacktrace=1"}, src=SHARE_SRC)


def test_host_helpers_random_tables_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                   "400", {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                           "UBSAN_OPTIONS": "print_stacktrace=1"}, src=HOST_SRC)
