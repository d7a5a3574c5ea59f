"""The boundary from plain C: tests/c_client/decode_step_client.c includes
only rkv.h and the HIP runtime's C API, links librkv.so (and the oracle, to
check itself) and runs one decode step.  On the CPU the client must compile
as C11 and link; on the GPU it must run and match the oracle."""
import os
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_client", "decode_step_client.c")
LIB = os.path.join(ROOT, "sparse_kv_cache_hsa_amd", "librkv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_client(out_dir) -> str:
    if not os.path.exists(LIB):
        pytest.skip("librkv.so is not built")
    orc = oracle.build()
    exe = os.path.join(str(out_dir), "decode_step_client")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}",
           SRC, "-o", exe, LIB, orc, f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{os.path.dirname(LIB)}", f"-Wl,-rpath,{os.path.dirname(orc)}",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_client_compiles_and_links(tmp_path):
    exe = build_client(tmp_path)
    assert os.path.exists(exe)


@pytest.mark.gpu
def test_c_client_runs_a_decode_step(tmp_path):
    exe = build_client(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c client: ok" in r.stdout, r.stdout
