"""AddressSanitizer / UndefinedBehaviorSanitizer builds of host code, run on
the CPU.

* The fp64 oracle (forward and backward), built by gcc with the sanitizers,
  on small edge cases (tests/sanitize/oracle_driver.c).
* The host side of the library's C entry points and kernel dispatch
  (triattn_api.hip, kernel_mfma.hip compiled host-only, the launchers
  replaced by stubs that abort), driven with rejected, overflowing and empty
  arguments (tests/sanitize/abi_driver.cpp).

A sanitizer report aborts the driver; the test also checks that the same
flags do abort on a planted overflow, so a build that silently drops the
sanitizers cannot pass.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "masked_attention_tri_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
C_FLAGS = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, env=ENV, **kw)
    return r.returncode, r.stdout + r.stderr


def _need(tool):
    if not (shutil.which(tool) or os.path.exists(tool)):
        pytest.skip(f"{tool} not available")


def test_planted_overflow_is_caught(tmp_path):
    _need("gcc")
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint main(void){int *p = malloc(4 * sizeof(int));"
                   "p[4] = 1; int r = p[0]; free(p); return r & 0;}\n")
    exe = tmp_path / "bad"
    rc, out = _run(["gcc", *C_FLAGS, "-o", str(exe), str(src)])
    assert rc == 0, out
    rc, out = _run([str(exe)])
    assert rc != 0 and ("heap-buffer-overflow" in out or "runtime error" in out), out


@pytest.mark.parametrize("which", ["fwd", "bwd"])
def test_oracle_under_sanitizers(tmp_path, which):
    _need("gcc")
    src = os.path.join(ROOT, "oracle", "triattn_oracle.c" if which == "fwd" else "triattn_oracle_bwd.c")
    exe = tmp_path / f"oracle_{which}"
    defs = ["-DORACLE_BWD"] if which == "bwd" else []
    rc, out = _run(["gcc", "-std=c11", "-pthread", *C_FLAGS, *defs, "-o", str(exe),
                    os.path.join(SAN, "oracle_driver.c"), src, "-lm"])
    assert rc == 0, out
    rc, out = _run([str(exe)])
    assert rc == 0 and "oracle driver: ok" in out, out


def test_abi_host_validation_under_sanitizers(tmp_path):
    _need(HIPCC)
    _need(CLANGXX)
    objs = []
    for name in ("triattn_api", "kernel_mfma"):
        obj = tmp_path / f"{name}.o"
        rc, out = _run([HIPCC, "--offload-host-only", "-x", "hip", "-std=c++17", "-g", "-O1",
                        f"-I{ROOT}/include", "-Xarch_host", "-fsanitize=address,undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all", "-c",
                        os.path.join(CSRC, f"{name}.hip"), "-o", str(obj)])
        assert rc == 0, out
        objs.append(str(obj))
    for name in ("abi_driver", "launch_stubs"):
        obj = tmp_path / f"{name}.o"
        rc, out = _run([CLANGXX, "-std=c++17", *C_FLAGS, f"-I{ROOT}/include",
                        f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__", "-c",
                        os.path.join(SAN, f"{name}.cpp"), "-o", str(obj)])
        assert rc == 0, out
        objs.append(str(obj))
    exe = tmp_path / "abi"
    rc, out = _run([CLANGXX, "-fsanitize=address,undefined", "-o", str(exe), *objs,
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    assert rc == 0, out
    rc, out = _run([str(exe)])
    assert rc == 0 and "abi driver: ok" in out, out
