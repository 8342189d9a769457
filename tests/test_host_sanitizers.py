"""The host C and C++ code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU): the C oracle, the native block manager and the C ABI's
host-side argument checks are rebuilt with -fsanitize=address,undefined
(the HIP library's sanitizer flags apply to its host pass only) and their
pin and ABI tests are re-run against the sanitized builds in child
processes, with the matching sanitizer runtime preloaded.  Any report
aborts the child and fails the test.

  * gcc build of oracle/pagedkv_oracle.c: the oracle pins, the quantised
    oracle pins and the block-manager pins (tests/test_oracle_pins.py,
    tests/test_oracle_quant.py, tests/test_block_manager.py), with the
    native manager taken from a g++ build of csrc/block_manager.hip;
  * hipcc build of csrc/pagedkv_api.hip and csrc/block_manager.hip (host
    pass sanitized) linked with the normally built kernel objects: the C-ABI
    argument checks (tests/test_abi.py) and the native block manager again.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_attention_decode_scatter_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def gcc_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                       text=True).stdout.strip()
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


def clang_runtime():
    c = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return c[-1] if c else None


def run_child(code, preload, extra_env, tmp):
    script = os.path.join(tmp, "child.py")
    with open(script, "w") as f:
        f.write(code)
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **extra_env)
    r = subprocess.run([sys.executable, script], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    return r.stdout


CHILD_PINS = """
import ctypes, os, sys
sys.path.insert(0, {root!r})
from paged_attention_decode_scatter_amd import native as N
N._lib = ctypes.CDLL(os.environ["PKV_BM_SAN_LIB"])   # block manager only
N.status_string = lambda st: "status %d" % st         # lives in the HIP library
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider",
                      "tests/test_oracle_pins.py", "tests/test_oracle_quant.py",
                      "tests/test_block_manager.py",
                      "-k", "not test_native_argument_errors"]))   # status text: the clang run
"""

CHILD_ABI = """
import os, sys
sys.path.insert(0, {root!r})
from paged_attention_decode_scatter_amd import native as N
N.LIB_PATH = os.environ["PKV_SAN_LIB"]
N._lib = None
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py",
                      "tests/test_block_manager.py", "-k", "not only_declared and not oracle"]))
"""


def test_oracle_and_block_manager_under_gcc_sanitizers(tmp_path):
    rt = gcc_runtime()
    if rt is None or shutil.which("g++") is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    tmp = str(tmp_path)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    oracle = os.path.join(tmp, "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", *san, "-ffp-contract=off",
                    os.path.join(ROOT, "oracle", "pagedkv_oracle.c"), "-o", oracle, "-lm",
                    "-lpthread"], check=True)
    bm = os.path.join(tmp, "libbm_san.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", *san,
                    "-fvisibility=hidden", f"-I{INCLUDE}", "-x", "c++",
                    os.path.join(CSRC, "block_manager.hip"), "-o", bm], check=True)
    out = run_child(CHILD_PINS.format(root=ROOT), rt,
                    {"PKV_ORACLE_LIB": oracle, "PKV_BM_SAN_LIB": bm}, tmp)
    assert " passed" in out and "failed" not in out


def test_abi_checks_under_clang_sanitizers(tmp_path):
    rt = clang_runtime()
    hipcc = "/opt/rocm/bin/hipcc"
    if rt is None or not os.path.exists(hipcc):
        pytest.skip("ROCm's clang AddressSanitizer runtime is not installed")
    from paged_attention_decode_scatter_amd import build

    kernels = [os.path.join(BUILD, s.replace(".hip", ".o"))
               for s in ("kernels_copy.hip", "kernels_decode.hip", "kernels_prefill.hip")]
    if not all(os.path.exists(k) for k in kernels):
        build.build()
    tmp = str(tmp_path)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              f"-I{INCLUDE}", f"-I{CSRC}"]
    api = os.path.join(tmp, "api.o")
    bm = os.path.join(tmp, "bm.o")
    subprocess.run([*common, *host_san, "-c", os.path.join(CSRC, "pagedkv_api.hip"), "-o", api],
                   check=True, capture_output=True)
    subprocess.run([*common, *host_san, "-c", os.path.join(CSRC, "block_manager.hip"), "-o", bm],
                   check=True, capture_output=True)
    lib = os.path.join(tmp, "libpagedkv_san.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san[:4], api, bm,
                    *kernels, "-o", lib], check=True, capture_output=True)
    out = run_child(CHILD_ABI.format(root=ROOT), rt, {"PKV_SAN_LIB": lib}, tmp)
    assert " passed" in out and "failed" not in out
