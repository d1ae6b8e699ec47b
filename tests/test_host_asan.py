"""The C-ABI host layer under AddressSanitizer, on the CPU.

fa_api.cpp (argument validation, workspace handling, dispatch) is built
with g++ -fsanitize=address and linked with host stand-ins for the HIP
runtime calls and kernel launchers (no device code).  The ABI and binding
tests then run against that build in a child process with the sanitizer
runtime preloaded, and a second child checks that the library-owned
workspace is released when the library is unloaded.
"""
import os
import re
import subprocess
import sys

import pytest

from exact_attention_116_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asan_env():
    try:
        lib = fabuild.build_host_asan()
        rt = fabuild.asan_runtime()
    except (RuntimeError, FileNotFoundError) as e:    # no g++ or no sanitizer runtime
        pytest.skip(f"no host AddressSanitizer toolchain: {e}")
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("the sanitizer runtime library was not found")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=97",
               PYTHONPATH=ROOT)
    return lib, env


def run_child(code, env):
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=300)


def test_abi_and_binding_tests_under_asan(asan_env):
    lib, env = asan_env
    code = (
        "import sys, pytest\n"
        "import exact_attention_116_amd as fa\n"
        f"fa.load({lib!r})\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
        "                      'tests/test_abi.py', 'tests/test_binding_sizes.py']))\n")
    r = run_child(code, env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert re.search(r"\d+ passed", r.stdout), r.stdout[-2000:]


def test_owned_workspace_released_at_unload(asan_env):
    """Decode and backward calls without a workspace grow the library-owned
    buffer (allocate, then free and reallocate when a call needs more); the
    buffer still held is freed when the library is unloaded."""
    lib, env = asan_env
    code = (
        "import ctypes, _ctypes, sys\n"
        f"lib = ctypes.CDLL({lib!r}, mode=ctypes.RTLD_LOCAL)\n"
        "A = 0x10000\n"
        "lib.fa_decode_splitkv.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 5\n"
        "assert lib.fa_decode_splitkv(A, A, A, A, 1, 2, 64, 128, 4) == 0\n"
        "assert lib.fa_decode_splitkv(A, A, A, A, 4, 8, 64, 128, 16) == 0\n"
        "print('calls done', flush=True)\n"
        "sys.stdout.flush()\n"
        "_ctypes.dlclose(lib._handle)\n"
        "print('unloaded', flush=True)\n")
    r = run_child(code, env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    mallocs = re.findall(r"stub hipMalloc \d+ -> (0x[0-9a-f]+)", r.stderr)
    frees = re.findall(r"stub hipFree (0x[0-9a-f]+)", r.stderr)
    assert len(mallocs) == 2, r.stderr       # grown once
    assert sorted(mallocs) == sorted(frees), r.stderr
    assert frees[-1] == mallocs[-1]           # the buffer in use went at unload
    assert "unloaded" in r.stdout
