"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only, no GPU code is sanitized).

1. The oracle (oracle/*.c) built by gcc with -fsanitize=address,undefined and loaded in place of
   the normal build (SAGE_ORACLE_LIB, gcc's libasan preloaded) runs the oracle's pin tests.
2. The C ABI's host layer (sage_api.cpp: argument validation, size queries, error paths) compiled
   by hipcc with the sanitizers on the host side only and linked with the library's kernel
   objects (clang's ASan runtime preloaded) runs the ABI tests, which call every entry point with
   invalid arguments, extreme sizes and unknown enum values.

Every finding aborts the child process (-fno-sanitize-recover=all, halt_on_error=1) and fails the
test with the sanitizer's report.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "SAGE_SANITIZER_CHILD": "1"}
# a child run never starts another one
pytestmark = pytest.mark.skipif(os.environ.get("SAGE_SANITIZER_CHILD") == "1", reason="inside a sanitizer run")


def _run_child(code: str, preload: str, extra_env: dict, logdir: str, timeout: int = 900):
    logdir = os.path.join(logdir, "sanitizer_logs")
    os.makedirs(logdir, exist_ok=True)
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **extra_env)
    env["ASAN_OPTIONS"] += f":log_path={logdir}/asan"
    env["UBSAN_OPTIONS"] += f":log_path={logdir}/ubsan"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    reports = ""
    for f in sorted(glob.glob(os.path.join(logdir, "*"))):
        with open(f) as fh:
            reports += fh.read()
    assert r.returncode == 0 and not reports, (
        f"exit {r.returncode}\n--- sanitizer reports ---\n{reports[-6000:]}\n--- output ---\n{r.stdout[-3000:]}"
        f"\n{r.stderr[-3000:]}")
    return r.stdout


@pytest.mark.slow
def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "libsage_oracle_san.so"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), asan
    files = sorted(glob.glob(os.path.join("tests", "test_oracle_*.py"))) + ["tests/test_golden_contracts.py"]
    code = ("import sys, pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-n', '4', "
            f"'-m', 'not gpu', *{files!r}]))")
    out = _run_child(code, asan, {"SAGE_ORACLE_LIB": lib}, str(tmp_path))
    assert " passed" in out


def _stale(objs, sources):
    newest = max(os.path.getmtime(s) for s in sources)
    return any(not os.path.exists(o) or os.path.getmtime(o) < newest for o in objs)


@pytest.mark.slow
def test_abi_host_layer_under_asan_ubsan(tmp_path):
    from quantized_attention_quantize_amd import build as B
    kernels = [s for s in B.SOURCES if s != "sage_api.cpp"]
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in kernels]
    headers = glob.glob(os.path.join(B.CSRC, "*.h")) + glob.glob(os.path.join(B.INCLUDE, "*.h"))
    if _stale(objs, [os.path.join(B.CSRC, s) for s in kernels] + headers):
        B.build_library()
    cc = B.hipcc()
    san = ["-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "sage_api_san.o")
    lib = str(tmp_path / "libsage_mi355x_san.so")
    subprocess.run([cc, *B.common_flags(), "-O1", "-g", *san, "-x", "hip", "-c",
                    os.path.join(B.CSRC, "sage_api.cpp"), "-o", api_o], check=True, capture_output=True)
    subprocess.run([cc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *san[:4], "-o", lib, api_o, *objs], check=True,
                   capture_output=True)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rt, "clang's ASan runtime is missing"
    code = ("import sys, pytest\n"
            "import quantized_attention_quantize_amd.api as a\n"
            f"a._LIB_PATH = {lib!r}\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi.py']))\n")
    out = _run_child(code, rt[0], {}, str(tmp_path))
    assert " passed" in out
