"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on a
host without a GPU: the scalar oracle (gcc build, libasan preloaded) runs
its pin tests, and the library's host code (hipcc build with the sanitizers
on the host side only, clang's ASan runtime preloaded) runs the expert pool's
policy tests in bookkeeping mode, each in a subprocess that fails on the
first report.

Pages: tech.takumi3488.com, "Trying colibri", the section on running the
unit tests and the quantisation self-test (the tier tests these mirror).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
MAPPED = ("import ctypes,sys; {load}; m=open('/proc/self/maps').read(); "
          "assert '{name}' in m, 'sanitized library not mapped'; "
          "ctypes.CDLL(None).__asan_init; print('sanitized library mapped')")


def run(env_extra, args, timeout=600):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    return r.stdout


def test_oracle_under_asan_ubsan():
    import oracle
    so = oracle.build(sanitize=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(libasan), "gcc's libasan not found"
    env = {"LD_PRELOAD": libasan, "MOE_ORACLE_LIB": so}
    run(env, ["-c", MAPPED.format(load="import oracle; oracle._load()", name=os.path.basename(so))])
    out = run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle_quant.py",
                    "tests/test_oracle_router.py", "tests/test_oracle_ffn.py", "tests/test_oracle_topp.py"])
    assert " passed" in out and "failed" not in out


def test_pool_host_code_under_asan_ubsan():
    from quantized_moe_expert_sigmoid_amd import build
    so = build.build(force=False, sanitize=True)
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    env = {"LD_PRELOAD": rt[-1], "MOE_LIBRARY": so}
    run(env, ["-c", MAPPED.format(load="import quantized_moe_expert_sigmoid_amd as m; m.lib()",
                                  name=os.path.basename(so))])
    out = run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_pool_cpu.py",
                    "tests/test_pool_tiers_cpu.py"])
    assert " passed" in out and "failed" not in out
