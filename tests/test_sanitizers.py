"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The oracle (oracle/ffd_oracle.c) is built with -fsanitize=address,undefined into a temporary
   directory, and its whole pin suite (tests/test_oracle_*.py) runs against that build in a
   subprocess with the ASan runtime preloaded.
2. The C-ABI layer (long_context_decoding_amd/csrc/ffd_api.cpp: validation, split heuristic,
   workspace layout) is built host-only with g++ and the same sanitizers, its kernel launchers
   replaced by counting stubs (tests/sanitize/launch_stubs.cpp); tests/test_abi.py runs against it,
   then a set of valid calls that reach the (stub) launchers, and every launching entry point
   once more with its launch made to fail, which must return FFD_ERR_HIP.

Any sanitizer report aborts the subprocess (halt_on_error, no recovery), which fails the test.  A
negative control checks that the harness does report a planted heap overflow.
"""
import os
import shutil
import subprocess
import sys
import textwrap
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ORACLE_TESTS = sorted(str(p) for p in (ROOT / "tests").glob("test_oracle_*.py"))


def _asan_runtime() -> str | None:
    if not shutil.which("gcc"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


ASAN = _asan_runtime()
pytestmark = pytest.mark.skipif(ASAN is None or not shutil.which("g++"),
                                reason="gcc/g++ with libasan not available")


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = ASAN
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = os.pathsep.join([str(ROOT), str(ROOT / "tests")])
    return env


def _run(script: str, timeout: int = 600) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, "-c", textwrap.dedent(script)], cwd=ROOT, env=_env(),
                          capture_output=True, text=True, timeout=timeout)


def _assert_clean(res: subprocess.CompletedProcess):
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "libffd_oracle_san.so"
    subprocess.run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", "-Wall", "-o", str(lib), str(ROOT / "oracle" / "ffd_oracle.c"),
                    "-lm"], check=True)
    res = _run(f"""
        import sys
        from pathlib import Path
        import oracle
        oracle._LIB_PATH = Path({str(lib)!r})
        import pytest
        rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", *{ORACLE_TESTS!r}])
        assert {str(lib)!r} in open("/proc/self/maps").read(), "sanitized oracle not loaded"
        sys.exit(int(rc))
    """)
    _assert_clean(res)
    assert " passed" in res.stdout


def test_abi_layer_under_sanitizers(tmp_path):
    lib = tmp_path / "libffd_host_san.so"
    subprocess.run(["g++", "-std=c++17", *SAN, "-fPIC", "-shared", "-Wall",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-o", str(lib),
                    str(ROOT / "long_context_decoding_amd" / "csrc" / "ffd_api.cpp"),
                    str(ROOT / "tests" / "sanitize" / "launch_stubs.cpp")], check=True)
    res = _run(f"""
        import ctypes, sys
        from pathlib import Path
        from long_context_decoding_amd import ffd
        ffd.LIB_PATH = Path({str(lib)!r})
        import pytest
        rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py", "-k",
                          "not probe"])
        if rc != 0:
            sys.exit(int(rc))
        L = ffd.lib()
        n = ctypes.CDLL({str(lib)!r}).ffd_stub_launches
        # every call of the ABI suite is rejected or has nothing to launch
        assert n() == 0, n()
        A = ctypes.c_void_p(1 << 16)
        for B, Hq, Hkv, Lt, T in ((1, 32, 8, 262144, 128), (8, 32, 8, 131072, 64),
                                  (2, 28, 4, 4096 + 17, 64), (1, 64, 4, 32768, 64),
                                  (3, 9, 1, 100, 64), (1, 1, 1, 1, 128)):
            d = ffd.make_dims(B, Hq, Hkv, Lt, -(-Lt // T) * T, ffd.FFD_BF16)
            ws = ffd.workspace_bytes(d, T)
            assert ws > 0
            before = n()
            assert L.ffd_decode_sparse(ctypes.byref(d), A, A, A, A, A, 5.0, T, A, A, A, A, ws,
                                       None) == 0
            assert L.ffd_decode_dense(ctypes.byref(d), A, A, A, T, A, A, A, ws, None) == 0
            assert L.ffd_decode_masked(ctypes.byref(d), A, A, A, A, T, A, A, A, ws, None) == 0
            assert L.ffd_decode_sparse_running(ctypes.byref(d), A, A, A, A, A, 5.0, T, 8, A, A,
                                               None, A, 1 << 40, None) in (0, 2)
            assert L.ffd_quantize_k_append(ctypes.byref(d), A, 0, Lt, T, A, A, None) == 0
            assert L.ffd_workspace_init(ctypes.byref(d), T, A, ws, None) == 0
            assert L.ffd_block_scores(ctypes.byref(d), 0, A, A, A, A, A, A, T, A, None) == 0
            assert L.ffd_select_blocks(ctypes.byref(d), 1, A, None, 3.0, T, A, None) in (0, 2)
            assert L.ffd_decode_sparse_noalloc(ctypes.byref(d), A, A, A, A, A, 5.0, T, A, A,
                                               None, None) in (0, 3)
            assert n() > before
        # every launching entry point maps a failed launch (or scratch-area lookup) to
        # FFD_ERR_HIP, and the failure does not stick to the next call
        fail = ctypes.CDLL({str(lib)!r}).ffd_stub_fail_next
        T = 128
        d = ffd.make_dims(1, 32, 8, 4096, 4096, ffd.FFD_BF16)
        ws = ffd.workspace_bytes(d, T)
        D = ctypes.byref(d)
        calls = {{
            "decode_sparse": lambda: L.ffd_decode_sparse(D, A, A, A, A, A, 5.0, T, A, A, A, A, ws, None),
            "decode_dense": lambda: L.ffd_decode_dense(D, A, A, A, T, A, A, A, ws, None),
            "decode_masked": lambda: L.ffd_decode_masked(D, A, A, A, A, T, A, A, A, ws, None),
            "decode_sparse_running": lambda: L.ffd_decode_sparse_running(
                D, A, A, A, A, A, 5.0, T, 8, A, A, None, A, 1 << 40, None),
            "decode_sparse_noalloc": lambda: L.ffd_decode_sparse_noalloc(
                D, A, A, A, A, A, 5.0, T, A, A, None, None),
            "decode_sparse_residual": lambda: L.ffd_decode_sparse_residual(
                D, A, None, A, A, A, A, A, 2, 5.0, T, A, A, None, A, ws, None),
            "decode_sparse_varlen": lambda: L.ffd_decode_sparse_varlen(
                D, A, A, A, A, A, A, 5.0, T, A, A, None, A, ws, None),
            "decode_dense_varlen": lambda: L.ffd_decode_dense_varlen(D, A, A, A, A, T, A, A, A, ws, None),
            "decode_sparse_append": lambda: L.ffd_decode_sparse_append(
                D, A, A, A, A, A, A, A, A, 5.0, T, A, A, None, A, ws, None),
            "quantize_k_append": lambda: L.ffd_quantize_k_append(D, A, 0, 4096, T, A, A, None),
            "quantize_k_residual_append": lambda: L.ffd_quantize_k_residual_append(
                D, A, 0, 4096, T, 2, A, A, A, A, None),
            "append_token": lambda: L.ffd_append_token(D, A, A, A, A, A, T, A, A, None),
            "workspace_init": lambda: L.ffd_workspace_init(D, T, A, ws, None),
            "block_bounds": lambda: L.ffd_block_bounds(D, A, 0, 4096, T, A, A, None),
            "block_scores": lambda: L.ffd_block_scores(D, 0, A, A, A, A, A, A, T, A, None),
            "select_blocks": lambda: L.ffd_select_blocks(D, 1, A, None, 3.0, T, A, None),
        }}
        for name, call in calls.items():
            assert call() == 0, (name, "with working launches")
            fail(1)
            assert call() == 4, (name, "with a failed launch")
            assert call() == 0, (name, "after a failed launch")
        sys.exit(0)
    """)
    _assert_clean(res)


def test_harness_reports_a_planted_overflow(tmp_path):
    """Negative control: a library that reads past a heap buffer must make the subprocess fail
    with an AddressSanitizer report under the same preload and options."""
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int read_past(int n) { int* a = (int*)malloc(sizeof(int) * n);\n"
                   "  for (int i = 0; i < n; ++i) a[i] = i;\n"
                   "  int v = a[n]; free(a); return v; }\n")
    lib = tmp_path / "liboverflow.so"
    subprocess.run(["gcc", *SAN, "-fPIC", "-shared", "-o", str(lib), str(src)], check=True)
    res = _run(f"""
        import ctypes
        ctypes.CDLL({str(lib)!r}).read_past(8)
    """, timeout=120)
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr
