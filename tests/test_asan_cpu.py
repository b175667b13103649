"""The library's host code under AddressSanitizer, on the CPU.

`paged_kv_cache_14_amd.build.build_asan_library` compiles the host side of
every source with -fsanitize=address; `tests/asan_driver.c`, linked with the
ASan runtime, drives the C ABI through its host-only paths: argument
validation of every entry point that enqueues work (all calls rejected before
any HIP call), workspace sizing, long random block-manager programs with
their invariants, and random batches through pa_check_batch.  Every buffer
the library touches is allocated at exactly its documented size, so an
overflow, a use after free or a leak fails the run.
"""
import os
import subprocess

import pytest

from paged_kv_cache_14_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "asan_driver.c")
CLANG = "/opt/rocm/llvm/bin/clang"


def _stale(target, inputs):
    return not os.path.exists(target) or \
        os.path.getmtime(target) < max(os.path.getmtime(p) for p in inputs)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm's clang is not installed")
    headers = [os.path.join(build.INCLUDE, h) for h in os.listdir(build.INCLUDE)]
    csrc_headers = [os.path.join(build.CSRC, h) for h in os.listdir(build.CSRC)
                    if h.endswith(".h")]
    if _stale(build.ASAN_LIB_PATH, build.sources() + headers + csrc_headers):
        build.build_asan_library()
    exe = str(tmp_path_factory.mktemp("asan") / "asan_driver")
    subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address",
                    "-fno-omit-frame-pointer", f"-I{build.INCLUDE}", DRIVER,
                    f"-L{build.ASAN_DIR}", "-lpa_asan", f"-Wl,-rpath,{build.ASAN_DIR}",
                    "-o", exe], check=True, capture_output=True, text=True)
    return exe


def test_host_code_is_clean_under_asan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1")
    res = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "asan driver: ok" in res.stdout
    assert "AddressSanitizer" not in res.stderr and "LeakSanitizer" not in res.stderr
