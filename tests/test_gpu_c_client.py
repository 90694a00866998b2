"""The C ABI from a plain C program (tests/c_client.c): hipMalloc'd buffers, a
HIP stream of its own, no Python binding and no torch, checked against the C
oracle. The program is compiled by the host C compiler against include/ssu.h
and the built library."""
import os
import subprocess

import pytest

from selective_state_update_ssu_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def compile_client(out_dir):
    lib_dir = os.path.dirname(build.LIBRARY)
    oracle_dir = os.path.join(ROOT, "oracle")
    exe = os.path.join(out_dir, "c_client")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{oracle_dir}",
           os.path.join(ROOT, "tests", "c_client.c"), "-o", exe,
           f"-L{lib_dir}", "-lssu_amd", f"-L{oracle_dir}", "-lssu_oracle",
           f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{lib_dir}:{oracle_dir}:{ROCM}/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_client_compiles(tmp_path):
    """The header and the library link from C (no GPU needed to build)."""
    if not os.path.exists(build.LIBRARY):
        pytest.skip("library not built")
    if not os.path.exists(os.path.join(ROOT, "oracle", "libssu_oracle.so")):
        pytest.skip("oracle not built")
    assert os.access(compile_client(str(tmp_path)), os.X_OK)


@pytest.mark.gpu
def test_c_client_matches_oracle(tmp_path):
    exe = compile_client(str(tmp_path))
    print("[c client] running", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c client ok" in r.stdout
