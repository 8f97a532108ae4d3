"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the library is rebuilt with both sanitizers on its host
compilation (argument checks, plan builder, launch set-up; the gfx950 code
is unchanged), and the host ABI tests and the plan-builder invariant tests
run against that build in a child process with the sanitizer runtime
preloaded. Any report fails the run."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from mla_paged_kv_02_amd import build as B
    lib = B.build(hostsan=True, out_path=str(tmp_path / "libmla_decode_hostsan.so"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms, "host code not built with AddressSanitizer"
    assert "__ubsan_handle" in syms, "host code not built with UndefinedBehaviorSanitizer"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": B.hostsan_runtime(),
        # the interpreter and torch are not instrumented: leaks at exit and
        # their own allocator pairing are not this library's
        "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:abort_on_error=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "MLA_DECODE_LIB": lib,
    })
    check_loaded = ("from mla_paged_kv_02_amd import _lib; import os; "
                    f"assert _lib.LIB_PATH == {lib!r}, _lib.LIB_PATH; _lib.lib()")
    r = subprocess.run([sys.executable, "-c", check_loaded], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi_host.py", "tests/test_sched_host.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]
