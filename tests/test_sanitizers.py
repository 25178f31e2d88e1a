"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* the oracle (oracle/vc_oracle.c) built with gcc -fsanitize=address,undefined runs its whole pin
  suite (tests/test_oracle_*.py, tests/test_golden_printed.py) with the gcc ASan runtime preloaded;
* the C ABI's host code (vc_api.hip: validation, aliasing checks, device check) built with the host
  pass instrumented (clang ASan/UBSan, kernels untouched) runs tests/test_abi.py with the clang
  runtime preloaded;
* a planted out-of-bounds read into the sanitized oracle must be reported, so a run that does not
  actually instrument anything cannot pass.
The sanitized libraries are built into a temporary directory and selected through VC_ORACLE_LIB
and VC_LIB_PATH; nothing here touches a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_asan():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _run(env_extra, args, timeout=900):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               PYTHONMALLOC="malloc", **env_extra)
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


@pytest.fixture(scope="module")
def libs(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("san"))
    import oracle
    ora = oracle.build(sanitize_to=os.path.join(d, "liboracle_san.so"))
    try:
        from bit_attention_video_online_amd import build_sanitized as bs
        vcl, rt = bs.build_sanitized(d), bs.asan_runtime()
    except Exception as e:  # no hipcc or no clang runtime: only the oracle part can run
        vcl, rt = None, repr(e)
    return dict(oracle=ora, vc=vcl, clang_rt=rt)


def test_oracle_pins_under_asan_ubsan(libs):
    tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_")) + ["tests/test_golden_printed.py"]
    r = _run({"LD_PRELOAD": _gcc_asan(), "VC_ORACLE_LIB": libs["oracle"]},
             ["-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"] + tests)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_abi_host_code_under_asan_ubsan(libs):
    if libs["vc"] is None:
        pytest.skip("sanitized ABI library not built: %s" % libs["clang_rt"])
    r = _run({"LD_PRELOAD": libs["clang_rt"], "VC_LIB_PATH": libs["vc"]},
             ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"])
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_planted_overflow_is_reported(libs):
    """Positive control: a decode call told to read 64 codes from a 16-byte array."""
    code = ("import ctypes, numpy as np, oracle\n"
            "a = np.zeros(16, np.uint8); o = np.zeros(64, np.float64)\n"
            "oracle.lib().or_e4m3_decode_array(a.ctypes.data_as(ctypes.c_void_p), "
            "o.ctypes.data_as(ctypes.c_void_p), 64)\n")
    r = _run({"LD_PRELOAD": _gcc_asan(), "VC_ORACLE_LIB": libs["oracle"]}, ["-c", code], timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
