"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (oracle/sqa_oracle.c), the input generator (inputs/gen.c) and the
argument checks of the C ABI (csrc/api.cpp with the host plans of
csrc/plan.cpp, kernel launchers replaced by recording stubs from
tests/sanitize) are built with -fsanitize=address,undefined into a
temporary folder.  The oracle pins, the generator tests, the checker
canaries and the ABI tests then run in a child pytest against those builds
(the loaders take the library paths from environment variables), with the
sanitizer runtime preloaded ahead of the interpreter's own libraries.  Any
sanitizer report fails the run.  A planted heap overflow checks that the
set-up really reports one.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fPIC", "-shared"]
ENV_OPTS = {
    # the interpreter and numpy keep memory until exit; only errors matter here
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1:alloc_dealloc_mismatch=0:"
                    "new_delete_type_mismatch=0:detect_odr_violation=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _libasan():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


def _env(libasan, extra):
    env = dict(os.environ)
    env.update(ENV_OPTS)
    env.update(extra)
    prev = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = libasan + (":" + prev if prev else "")
    return env


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    libasan = _libasan()
    if libasan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    d = tmp_path_factory.mktemp("san")
    oracle_so, inputs_so, abi_so = str(d / "liboracle.so"), str(d / "libinputs.so"), str(d / "libsqa_host.so")
    _run(["gcc"] + SAN + ["-fopenmp", os.path.join(ROOT, "oracle", "sqa_oracle.c"), "-o", oracle_so, "-lm"])
    _run(["gcc"] + SAN + ["-fopenmp", os.path.join(ROOT, "inputs", "gen.c"), "-o", inputs_so, "-lm"])
    csrc = os.path.join(ROOT, "reduced_query_head_amd", "csrc")
    _run(["g++"] + SAN + ["-std=c++17", "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                          os.path.join(csrc, "api.cpp"), os.path.join(csrc, "plan.cpp"),
                          os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", abi_so])
    return libasan, oracle_so, inputs_so, abi_so, d


def test_pins_generator_and_abi_checks_under_sanitizers(san_libs):
    libasan, oracle_so, inputs_so, abi_so, _ = san_libs
    env = _env(libasan, {"SQA_ORACLE_LIB": oracle_so, "SQA_INPUTS_LIB": inputs_so, "SQA_TEST_STUB_LIB": abi_so})
    files = ["tests/test_oracle_pins.py", "tests/test_inputs.py", "tests/test_checker_canaries.py", "tests/test_abi.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-6000:]
    # the stub-only ABI test ran (so the ABI tests really used the sanitized build)
    assert " skipped" not in out.splitlines()[-1], out.splitlines()[-1]


def test_planted_overflow_is_reported(san_libs):
    libasan, _, _, _, d = san_libs
    src = d / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted(int n) { int* a = malloc(n * sizeof(int)); a[n] = 1; int r = a[0]; free(a); return r; }\n")
    so = str(d / "libplanted.so")
    _run(["gcc"] + SAN + [str(src), "-o", so])
    code = f"import ctypes; ctypes.CDLL({so!r}).planted(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(libasan, {}), capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
