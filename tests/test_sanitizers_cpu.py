"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer over the C oracle and the C-ABI layer.

Builds instrumented copies of oracle/mmf_oracle.c (clang) and of the host code of
csrc/mmf_abi.hip (hipcc, the sanitizers on the host pass only; the kernels' objects are the
regular build's), then runs the CPU tests that exercise them -- the oracle pins and the ABI's
argument validation -- in a child process with the ASan runtime preloaded. Undefined behaviour
traps. No GPU is touched: the ABI tests stop at validation, before any HIP call.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
KERNEL_OBJECTS = ["k_quant", "k_scan", "k_contract", "k_bwd", "k_gemm_bf16", "k_generate", "k_ceiling", "k_hgrn2", "k_stack"]
SANITIZERS = ["-fsanitize=address", "-fsanitize=undefined", "-fsanitize-trap=undefined"]


def _asan_runtime():
    libs = sorted(glob.glob(ROCM + "/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(map(str, cmd)), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.timeout(900)
def test_oracle_and_abi_under_host_sanitizers(tmp_path):
    clang, hipcc, runtime = ROCM + "/llvm/bin/clang", ROCM + "/bin/hipcc", _asan_runtime()
    if not (runtime and os.path.exists(clang) and os.path.exists(hipcc)):
        pytest.skip("no ROCm clang with the ASan runtime")
    build = os.path.join(ROOT, "ternary_weight_matmul_amd", "_build")
    objs = [os.path.join(build, n + ".o") for n in KERNEL_OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built")

    oracle_so = str(tmp_path / "liboracle_san.so")
    _run([clang, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wno-unknown-pragmas"] + SANITIZERS + [os.path.join(ROOT, "oracle", "mmf_oracle.c"), "-o", oracle_so, "-lm"])

    host_only = []
    for flag in SANITIZERS:  # instrument the host pass only
        host_only += ["-Xarch_host", flag]
    abi_o = str(tmp_path / "mmf_abi_san.o")
    csrc = os.path.join(ROOT, "ternary_weight_matmul_amd", "csrc")
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"),
          "-I" + csrc, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-inline-asm"] + host_only +
         ["-c", os.path.join(csrc, "mmf_abi.hip"), "-o", abi_o])
    lib_so = str(tmp_path / "libmmf_san.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", SANITIZERS[0]] + objs + [abi_o, "-o", lib_so])

    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))) + [
        os.path.join(ROOT, "tests", "test_abi_cpu.py")]
    env = dict(os.environ, MMF_ORACLE_LIB=oracle_so, MMF_LIB=lib_so, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + tests,
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in r.stdout
