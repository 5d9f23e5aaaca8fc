"""The host part of the library (block tables, copy-on-write bookkeeping,
free queue, prefix cache) under AddressSanitizer and UndefinedBehaviorSanitizer.

The reference counting, copy-on-write and free-queue logic is the pages' core
bookkeeping (page "生成一个字，为什么要背一整本账", section
"PagedAttention：把操作系统的老智慧搬进推理引擎": blocks stored once,
reference counted, copied on write).  Here it is built with g++
-fsanitize=address,undefined as a host-only library, and the host tests (ABI
against the oracle's block manager, prefix cache against its oracle,
utilisation study, host benchmark) run against that build in a child
process with the sanitizer runtime preloaded; any report fails the test.  A
second child misuses the ABI on purpose (a capacity larger than the buffer)
to show that the sanitizer is live in that setup.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "paged_kv_cache_406_amd"))
import build as pkv_build  # noqa: E402

HOST_TESTS = ["tests/test_abi_host.py", "tests/test_prefix_cache.py", "tests/test_utilization.py",
              "tests/test_host_bench.py"]


def _env():
    if not shutil.which("g++"):
        pytest.skip("g++ not found")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not found")
    lib = pkv_build.build_host_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PKV_LIBRARY=lib,
               PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""))
    return env


def test_host_library_is_clean_under_asan_and_ubsan():
    env = _env()
    res = subprocess.run([sys.executable, "-m", "pytest", *HOST_TESTS, "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu and not device_code"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    passed = [l for l in out.splitlines() if " passed" in l]
    assert passed and int(passed[-1].split(" passed")[0].split()[-1]) >= 60, out[-2000:]


def test_sanitizer_reports_a_misused_buffer():
    env = _env()
    code = (
        "import ctypes, paged_kv_cache_406_amd as P\n"
        "from paged_kv_cache_406_amd import _binding as B\n"
        "h = P.kv_pool_create(P.make_desc(1, 1, 64, 4, 1000, 'f32'))\n"
        "s = P.block_table_alloc(h)\n"
        "P.block_table_append(h, s, 2800)\n"                      # 700 blocks
        "buf = (ctypes.c_int32 * 600)()\n"                        # a 2400-byte heap block
        "n, ln = ctypes.c_int32(), ctypes.c_int32()\n"
        "B._lib.block_table_get(h, s, buf, 700, ctypes.byref(n), ctypes.byref(ln))\n"   # cap overstated
        "print('not reported')\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode != 0 and "heap-buffer-overflow" in out and "block_table_get" in out, out[-3000:]
    assert "not reported" not in out
