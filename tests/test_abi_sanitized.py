"""The C-ABI argument checks (mask_aware_exact_amd/csrc/fm_api.hip) built for the host alone under
AddressSanitizer and UndefinedBehaviorSanitizer, linked against host-only stand-ins for the kernel
launchers (tests/sanitize/stub_launch.cpp) and driven through every entry point with valid and invalid
arguments (tests/sanitize/abi_check.cpp). CPU only: nothing is launched. Skipped when the ROCm compilers
are not installed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "mask_aware_exact_amd", "csrc")
ROCM = "/opt/rocm"


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_abi_checks_clean_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm compilers not installed")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17"]
    # host side only: each sanitizer flag applies to the host compilation
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    api_o = str(tmp_path / "fm_api.o")
    _run([hipcc, "--offload-arch=gfx950", "--offload-host-only", *flags, *inc, *host_san, "-c",
          os.path.join(CSRC, "fm_api.hip"), "-o", api_o])
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    objs = [api_o]
    for src in ("stub_launch.cpp", "abi_check.cpp"):
        o = str(tmp_path / src.replace(".cpp", ".o"))
        _run([clangxx, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), *flags, *inc, *san, "-c",
              os.path.join(SAN, src), "-o", o])
        objs.append(o)
    exe = str(tmp_path / "abi_check")
    _run([clangxx, *san, *objs, "-o", exe, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    assert "all expectations hold" in res.stdout
