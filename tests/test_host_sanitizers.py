"""Host-only checks of the library's host code (no GPU, no kernel launch):

* the ABI tests again, against a copy of the library whose host code is built
  with AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts);
* ttt_la_create when the workspace allocation fails: a preloaded stand-in for
  hipMalloc (tests/alloc_fail_shim.c) makes it fail with out-of-memory or with
  another HIP error, and the handle must come back NULL with TTT_LA_ERR_OOM or
  TTT_LA_ERR_HIP; a plan without workspace must not call hipMalloc at all.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from ttt_weight_layers_amd import build_sanitized  # noqa: E402


@pytest.fixture(scope="module")
def sanitized_lib():
    if build_sanitized.stale():
        build_sanitized.build()
    return build_sanitized.LIB


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        pytest.skip("no C compiler")
    out = str(tmp_path_factory.mktemp("shim") / "alloc_fail_shim.so")
    subprocess.run([cc, "-shared", "-fPIC", "-O1", "-o", out, os.path.join(ROOT, "tests", "alloc_fail_shim.c")],
                   check=True)
    return out


def _env(lib, preload):
    env = dict(os.environ)
    env["TTT_LA_LIBRARY"] = lib
    # keep whatever the environment already preloads, after ours
    env["LD_PRELOAD"] = ":".join(p for p in preload + [os.environ.get("LD_PRELOAD", "")] if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT
    return env


def test_library_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", "-D", sanitized_lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_abi_suite_under_sanitizers(sanitized_lib):
    env = _env(sanitized_lib, [build_sanitized.runtime()])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_zz_no_alloc.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail


CREATE = textwrap.dedent("""
    import ctypes, sys
    import ttt_weight_layers_amd as tla
    shim = ctypes.CDLL(None)
    shim.alloc_fail_shim_calls.restype = ctypes.c_int
    B, H, T, d, dtype = (int(a) if a.isdigit() else a for a in sys.argv[1:6])
    st, h = tla.ttt_la_create(tla.make_desc(B, H, T, d, d, dtype=dtype))
    print(st, h.value is None, shim.alloc_fail_shim_calls())
    if h.value is not None:
        tla.ttt_la_destroy(h)
""")


def _create(lib, preload, shape, status=None):
    env = _env(lib, preload)
    if status is not None:
        env["ALLOC_FAIL_STATUS"] = str(status)
    r = subprocess.run([sys.executable, "-c", CREATE, *map(str, shape)], env=env, capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    st, null, calls = r.stdout.split()[-3:]
    return int(st), null == "True", int(calls)


# bf16 at d = 128 over 4096 tokens: a segmented plan with a workspace
WITH_WS = (1, 2, 4096, 128, "bf16")
# fp32: the plan without workspace
NO_WS = (1, 2, 256, 64, "f32")


@pytest.mark.parametrize("sanitized", [False, True])
def test_create_reports_out_of_memory(sanitized, sanitized_lib, shim):
    import ttt_weight_layers_amd as tla
    lib = sanitized_lib if sanitized else tla.LIB_PATH
    pre = ([build_sanitized.runtime()] if sanitized else []) + [shim]
    st, null, calls = _create(lib, pre, WITH_WS)
    assert (st, null, calls) == (tla.TTT_LA_ERR_OOM, True, 1)
    st, null, calls = _create(lib, pre, WITH_WS, status=1)   # hipErrorInvalidValue
    assert (st, null, calls) == (tla.TTT_LA_ERR_HIP, True, 1)
    st, null, calls = _create(lib, pre, NO_WS)
    assert (st, null, calls) == (tla.TTT_LA_OK, False, 0)
