"""The host side of the library (argument checks, schedule planners, the C ABI) under
AddressSanitizer and UndefinedBehaviorSanitizer: the library is rebuilt with both on its host
code, and the CPU ABI tests run against it in a child process that preloads the sanitizer
runtime.  Any out-of-bounds access, use after free, signed overflow, bad shift or misaligned
access in those paths stops the child with a report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "sparse_query_sdpa_amd"))

CHILD = """
import sys
import sparse_query_sdpa_amd as sq
maps = open('/proc/self/maps').read()
assert sq.LIB_PATH == {lib!r}, sq.LIB_PATH
assert 'libclang_rt.asan' in maps and 'libsafe_hostsan.so' in maps, 'sanitized library or runtime not mapped'
import pytest
sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', {tests!r}]))
"""


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="the HIP toolchain is needed to build the sanitized library")
def test_abi_checks_are_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    import build
    lib = build.build_host_sanitized(str(tmp_path / "hostsan"))
    env = dict(os.environ)
    env.update({
        "SAFE_LIB_PATH": lib,
        "LD_PRELOAD": build.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",   # host paths only, also where a GPU is present
    })
    code = CHILD.format(lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
