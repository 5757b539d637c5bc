"""The host C++ (block manager, scheduler, error text) built with
AddressSanitizer and UndefinedBehaviorSanitizer, exercised by the host tests
in a child process (CPU only; see kv_cache_compression_paged_amd/host_sanitize.py).

The child runs the scheduler tests (native scheduler against the reference
model on every workload, bad-use errors) and the block-manager tests (random
histories against the oracle, error paths, shared-block refusal); any
sanitizer report aborts it.
"""

import shutil

import pytest


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_is_clean_under_asan_and_ubsan():
    from kv_cache_compression_paged_amd import host_sanitize
    r = host_sanitize.run(["tests/test_scheduler.py", "tests/test_abi_host.py",
                           "-k", "scheduler or block_manager"])
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_the_child_loads_the_sanitized_build():
    import os
    import subprocess
    import sys
    from kv_cache_compression_paged_amd import host_sanitize
    lib = host_sanitize.build()
    env = dict(os.environ, ZIPAGE_LIB=lib, LD_PRELOAD=":".join(host_sanitize.runtime_libs()),
               ASAN_OPTIONS="detect_leaks=0")
    out = subprocess.run([sys.executable, "-c",
                          "import kv_cache_compression_paged_amd as Z; "
                          "print(Z.lib()._name); print(Z.BlockManager(4).free_count())"],
                         cwd=host_sanitize.ROOT, env=env, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr[-2000:]
    name, count = out.stdout.split()
    assert name == lib and count == "4"
