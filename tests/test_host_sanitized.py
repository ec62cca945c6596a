"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds libslora with its host code instrumented (rank_gemm_page_amd.build.
build_sanitized; device code as usual) and runs the host-library tests
against it in a child process with the sanitizer runtime preloaded: the page
allocator and block table, adapter images, the segment builder and tile
lists on the five benchmark batches, and every argument-error path.  Any
out-of-bounds access, use after free or undefined behaviour aborts the child
and fails this test.  No GPU is used.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib):
    if not os.path.exists(lib):
        return True
    csrc = os.path.join(ROOT, "rank_gemm_page_amd", "csrc")
    newest = max(os.path.getmtime(os.path.join(d, f)) for d in (csrc, os.path.join(ROOT, "include"))
                 for f in os.listdir(d))
    return os.path.getmtime(lib) < newest


def test_host_library_clean_under_asan_and_ubsan():
    from rank_gemm_page_amd.build import SANITIZED_LIB_PATH, asan_runtime, build_sanitized
    if _stale(SANITIZED_LIB_PATH):
        build_sanitized()
    runtime = asan_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, LD_PRELOAD=runtime, SLORA_LIB=SANITIZED_LIB_PATH,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # every host test, the tile-coverage sweep on two of its routes
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_host_lib.py"), "-x", "-q",
           "-p", "no:cacheprovider", "-k", "not cover_each_output_once or default or all_mfma"]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
