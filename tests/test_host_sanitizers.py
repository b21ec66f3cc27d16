"""The host side of the C-ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

Builds the library with vdn_host.hip instrumented on its host pass -- the
argument checks, the per-entry workspace carving, the host loops of
vdn_window_plan and vdn_window_row_keys -- and runs the C-ABI test module
against it in a child process (the shared ASan runtime preloaded, any report
fatal).  Every call there is rejected before its first HIP call or touches
no device, so the whole module runs on a host without a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_module_clean_under_asan_and_ubsan(tmp_path):
    from softmax_attention_video_amd import _build as B
    try:
        lib = B.build_sanitized(str(tmp_path / "san"))
        rt = B.asan_runtime()
    except RuntimeError as e:     # no HIP compiler / sanitizer runtime on this host
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, VDN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
