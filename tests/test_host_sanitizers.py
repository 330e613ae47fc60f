"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: a copy of the library whose host code at the ABI (argument
checks, workspace carving, launch set-up) is instrumented runs every test of
test_abi_cpu.py (bad arguments of every entry point, sizes, version,
exports) in a child process with the ASan runtime preloaded; any invalid
access or undefined behaviour aborts that process.  Device code is not
instrumented and nothing runs on a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not found")
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("the ASan runtime of ROCm clang is not installed")
    return rt


def test_abi_checks_under_host_sanitizers(tmp_path):
    rt = _asan_runtime()
    from packed_bit_grouped_amd import build
    lib = build.build_host_check(str(tmp_path / "libmoe_w4_host_check.so"))
    # the entry points are instrumented (ASan report hooks referenced)
    syms = subprocess.run(["nm", "-u", os.path.join(build.HERE, "_build", "host_check",
                                                    "api.cpp.o")],
                          capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            "from packed_bit_grouped_amd import _lib as L\n"
            f"L.load({lib!r})\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    env = {**os.environ, "LD_PRELOAD": rt, "ASAN_OPTIONS": "detect_leaks=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    assert " passed" in r.stdout, out
