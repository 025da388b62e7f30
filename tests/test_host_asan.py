"""Host-side AddressSanitizer leg of the CPU tier.

The library's host code (the C ABI in api.hip: argument validation,
workspace arithmetic, launch set-up) is rebuilt with AddressSanitizer on the
host pass only (the gfx950 code objects are the ordinary ones), and every
call of the boundary tests runs against that build in a child process with
the ASan runtime preloaded.  A heap or stack error aborts the child with the
sanitizer's report.  No GPU is involved: the boundary calls are built to
fail validation before anything is launched.
"""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_script():
    path = os.path.join(ROOT, "causal_softmax_attention_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_attn_build_asan", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_boundary_calls_are_clean_under_host_asan(tmp_path):
    b = _build_script()
    try:
        runtime = b.asan_runtime()
        b.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = b.build_asan()
    pkg = tmp_path / "causal_softmax_attention_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "causal_softmax_attention_amd", "__init__.py"), pkg)
    shutil.copy(lib, pkg / "libattn.so")
    boundary = os.path.join(ROOT, "tests", "test_boundary.py")
    runner = (
        "import sys\n"
        f"sys.path.insert(0, {str(tmp_path)!r}); sys.path.insert(1, {ROOT!r})\n"
        "import causal_softmax_attention_amd as A\n"
        f"assert A.lib_path().startswith({str(tmp_path)!r}), A.lib_path()\n"
        "import pytest\n"
        f"sys.exit(pytest.main([{boundary!r}, '-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu']))\n")
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:exitcode=23:verify_asan_link_order=0")
    r = subprocess.run([sys.executable, "-c", runner], env=env, cwd=str(tmp_path), capture_output=True,
                       text=True, timeout=900)
    report = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
