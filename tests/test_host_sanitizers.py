"""The host layer under AddressSanitizer and UndefinedBehaviorSanitizer: the
CPU suites of the C ABI (argument checks, workspace sizing, error strings,
validators) and of the block manager (hand-worked cases, copy-on-write,
4,000 seeded operations against the model) run in a child process against
libpa_host_san.so -- api.cpp and block_manager.cpp built by g++ with both
sanitizers, any finding fatal, device side stubbed out
(paged_kv_cache_237_amd/build_host_san.py; __graft_entry__.build() builds it).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "paged_kv_cache_237_amd", "libpa_host_san.so")


def _runtime() -> str:
    """g++'s AddressSanitizer runtime, to preload into the child python."""
    try:
        p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                           text=True).stdout.strip()
    except OSError:
        return ""
    return p if os.path.isabs(p) and os.path.exists(p) else ""


RUNTIME = _runtime()

pytestmark = pytest.mark.skipif(not os.path.exists(SAN_LIB) or not RUNTIME,
                                reason="sanitizer build of the host layer not built, or no libasan")


def _env():
    return dict(os.environ, PA_LIB_PATH=SAN_LIB, LD_PRELOAD=RUNTIME,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def test_sanitizer_runtime_is_live_in_the_child():
    """The child loads the sanitized library with the ASan runtime mapped, and
    the library's code is instrumented (it calls the ASan and UBSan hooks)."""
    code = ("import paged_kv_cache_237_amd as pa; pa.lib(); "
            "print(pa.LIB_PATH); print(open('/proc/self/maps').read().count('libasan'))")
    r = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    path, maps = r.stdout.split()[-2:]
    assert path == SAN_LIB and int(maps) > 0
    nm = subprocess.run(["nm", "-D", "--undefined-only", SAN_LIB], capture_output=True,
                        text=True).stdout
    assert "__asan_report_" in nm and "__ubsan_handle_" in nm


def test_abi_and_block_manager_suites_run_clean():
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_block_manager.py"],
                       env=_env(), capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    assert " passed" in r.stdout and "failed" not in r.stdout, out
