"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU: the oracle (its pin tests, with the oracle built
with both sanitizers) and the C ABI's host code (the ABI tests, against the library built with both sanitizers on its
host code). Each run is a child process that preloads the sanitizer runtime its build needs; any report aborts it.
Nothing here touches a GPU."""
import ctypes
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
ENV_BASE = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "PYTHONDONTWRITEBYTECODE": "1"}


def gcc_asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return os.path.realpath(path) if os.path.isabs(path) and os.path.exists(path) else None


def run_child(args, preload, extra_env):
    env = dict(os.environ)
    env.update(ENV_BASE)
    env.update(extra_env)
    env["LD_PRELOAD"] = preload
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module")
def oracle_san(tmp_path_factory):
    import oracle
    rt = gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return oracle.build_sanitized(str(tmp_path_factory.mktemp("san") / "liboracle_san.so")), rt


def test_oracle_sanitizer_is_live(oracle_san):
    """A write past the end of an output array inside the sanitized oracle is reported and ends the process (the
    mistake is made by this test's call, on the CPU)."""
    lib, rt = oracle_san
    code = ("import ctypes, numpy as np\n"
            f"L = ctypes.CDLL({lib!r})\n"
            "v = np.zeros(64)\n"
            "out = np.zeros(8, dtype=np.uint16)\n"
            "L.orc_bf16_round_array(ctypes.c_void_p(v.ctypes.data), ctypes.c_int64(64), "
            "ctypes.c_void_p(out.ctypes.data))\n"
            "print('not reported')\n")
    r = run_child(["-c", code], rt, {})
    assert r.returncode != 0 and "not reported" not in r.stdout
    assert "AddressSanitizer" in r.stderr


def test_oracle_pins_under_sanitizers(oracle_san):
    """Every oracle pin test, with the oracle built with both sanitizers."""
    lib, rt = oracle_san
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    r = run_child(["-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests], rt,
                  {"QERL_ORACLE_LIB": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout


@pytest.fixture(scope="module")
def host_san():
    from nvfp4_weight_only_amd import build_lib
    rt = build_lib.sanitizer_runtime()
    if not rt:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    return build_lib.build_host_sanitized(), rt


def test_abi_host_code_under_sanitizers(host_san):
    """The ABI tests (host validation of every entry point, workspace queries and kernel plans over many shapes and
    options, exports) against the library built with both sanitizers on its host code."""
    lib, rt = host_san
    r = run_child(["-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                   os.path.join(ROOT, "tests", "test_abi.py")], rt, {"QERL_NVFP4_LIB": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout


def test_abi_sanitizer_is_live(host_san):
    """The sanitized library's host code reports a bad read: a projection array shorter than the count passed reads
    past its end (the mistake is made by this test's call, on the CPU; validation fails before any launch)."""
    lib, rt = host_san
    code = ("import ctypes, numpy as np\n"
            f"L = ctypes.CDLL({lib!r})\n"
            "L.nvfp4_lora_linear_workspace.restype = ctypes.c_size_t\n"
            "buf = np.zeros(16, dtype=np.uint8)\n"  # far smaller than one projection descriptor
            "print(L.nvfp4_lora_linear_workspace(ctypes.c_int64(16), ctypes.c_int64(256), "
            "ctypes.c_void_p(buf.ctypes.data), ctypes.c_int32(3)))\n"
            "print('not reported')\n")
    r = run_child(["-c", code], rt, {})
    assert r.returncode != 0 and "not reported" not in r.stdout
    assert "AddressSanitizer" in r.stderr
