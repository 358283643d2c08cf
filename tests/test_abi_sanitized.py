"""The host paths of the library (argument checks, planning, workspace sizing, error strings)
under AddressSanitizer and UndefinedBehaviorSanitizer: the CPU ABI tests re-run in a child
process against the host-sanitized build, with the ASan runtime preloaded. No GPU is touched."""
import os
import subprocess
import sys

import pytest

from compressed_sparse_kv_03_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_asan_ubsan():
    rt = build_lib.asan_runtime()
    if rt is None:
        pytest.skip("no shared ASan runtime next to hipcc")
    lib = build_lib.build_sanitized(verbose=False)
    env = dict(os.environ)
    env["CSKV_LIB_PATH"] = lib
    # the ASan runtime must come first; anything already preloaded stays
    env["LD_PRELOAD"] = ":".join([rt] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out and "failed" not in out, out[-2000:]
