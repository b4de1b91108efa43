"""The oracle pins and the host-side argument checks of the C ABI, run once
more under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Both the oracle and the library's host code are rebuilt with the
sanitizers (the library's device code is untouched), clang's ASan runtime is
preloaded, and the CPU tests of the oracle, the ABI checks and the binding
checks run in a child pytest against those builds; any finding aborts the
child and fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_checks_and_oracle_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle
    from mamba_ssd_scan_chunk_amd import build

    lib = build.build_host_sanitized(str(tmp_path / "lib"))
    olib = oracle.build_sanitized(str(tmp_path / "libssd_oracle_asan.so"))
    for so in (lib, olib):  # both builds really are instrumented
        syms = subprocess.check_output(["nm", "-D", so], text=True)
        assert "__asan_report" in syms and "__ubsan_handle" in syms, so
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": build.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "SSD_LIB_PATH": lib,
        "SSD_ORACLE_LIB": olib,
    })
    tests = ["tests/test_oracle_pins.py", "tests/test_abi_host.py", "tests/test_binding_host.py",
             "tests/test_zz_no_alloc.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-m", "not gpu", "-q", "-s", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    passed = int(r.stdout.strip().splitlines()[-1].split(" passed")[0].split()[-1])
    assert passed > 200, tail
