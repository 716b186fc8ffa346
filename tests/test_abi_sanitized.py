"""The library's host code (argument validation and workspace sizing in
convrot_api.hip) built with AddressSanitizer and UndefinedBehaviorSanitizer
on the host side only, linked with the unchanged kernel objects, and driven
by tests/sanitize_abi.c on the CPU: every sizing query over a grid of shapes
(extremes included) and every validation path that returns before a launch.
An out-of-bounds access, an integer overflow or other undefined behaviour in
that code fails here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
BUILD = os.path.join(ROOT, "_build")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    from w8a8_int8_rotated_amd import build as hb
    kernels = [os.path.join(BUILD, f) for f in ("gemm_i8.hip.o", "rotquant.hip.o", "probes.hip.o")]
    if not all(os.path.exists(k) for k in kernels):
        pytest.fail("kernel objects not built (run __graft_entry__.build())")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = tmp_path / "convrot_api.o"
    flags = [f for f in hb.COMMON if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([HIPCC, *flags, *san, "-c",
                        os.path.join(ROOT, "w8a8_int8_rotated_amd", "csrc", "convrot_api.hip"),
                        "-o", str(api_o)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = tmp_path / "libconvrot.so"
    r = subprocess.run([HIPCC, f"--offload-arch={hb.ARCH}", "-shared", "-fPIC",
                        "-fsanitize=address,undefined", str(api_o), *kernels, "-o", str(lib)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "sanitize_abi"
    r = subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", f"-I{ROOT}/include",
                        os.path.join(ROOT, "tests", "sanitize_abi.c"), str(lib),
                        f"-Wl,-rpath,{tmp_path}", f"-L{ROCM}/lib", "-lamdhip64",
                        f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the HIP runtime keeps allocations for the life of the process: leak
    # reports would be its, not this library's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert " 0 failed checks" in r.stdout
