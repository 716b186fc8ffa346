"""The C ABI used from C alone (tests/c_abi_forward.c): built with gcc
against include/convrot.h, libconvrot.so and libamdhip64, with the C oracle
linked beside it.  The build is checked on the CPU; the run needs the GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "w8a8_int8_rotated_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out):
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           os.path.join(ROOT, "tests", "c_abi_forward.c"),
           os.path.join(ROOT, "oracle", "convrot_oracle.c"),
           f"-L{PKG}", "-lconvrot", f"-Wl,-rpath,{PKG}",
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-lm", "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_c_program_builds(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libconvrot.so")):
        pytest.fail("libconvrot.so not built (run __graft_entry__.build())")
    assert os.path.exists(_build(tmp_path / "c_abi_forward"))


@pytest.mark.gpu
def test_c_program_forward_matches_oracle(tmp_path):
    exe = _build(tmp_path / "c_abi_forward")
    print("[case] C program: prepare + linear forward, padded low-rank pairs and the SwiGLU MLP "
          "through the C ABI",
          flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout.strip(), r.stderr.strip(), flush=True)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stdout}{r.stderr}"
    assert "0 codes, 0 scales, 0 outputs differ" in r.stdout
    assert r.stdout.count("0 outputs differ from the oracle") == 4
