"""The boundary is a C ABI: include/eidm.h compiles as strict C11 and as
C++17, and a plain C program linked against libeidm.so makes host-only calls
(ABI version, a query of the decode shape, a rejected query with its error
text).  Needs gcc/g++ and the built library; no GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "expert_id_matmul_amd")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def test_header_compiles_as_strict_c_and_cpp(tmp_path):
    _need("gcc")
    _need("g++")
    src = tmp_path / "h.c"
    src.write_text('#include "eidm.h"\nint eidm_header_probe(void) { return EIDM_ROUTE_GROUPED; }\n')
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, "-c", str(src),
                    "-o", str(tmp_path / "h_c.o")], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-pedantic", "-x", "c++", "-I", INCLUDE,
                    "-c", str(src), "-o", str(tmp_path / "h_cpp.o")], check=True)


def test_plain_c_program_calls_the_library(tmp_path):
    _need("gcc")
    lib = os.path.join(LIBDIR, "libeidm.so")
    if not os.path.exists(lib):
        pytest.skip("libeidm.so is not built")
    exe = tmp_path / "c_abi_host"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE,
                    os.path.join(HERE, "c_abi_host.c"), "-L", LIBDIR, "-leidm", f"-Wl,-rpath,{LIBDIR}", "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.splitlines()
    assert out[0] == "abi 2"
    # decode: AUTO picks Direct; the pages' extent (E-1)*stride + n*k*size; m*top_k*n outputs
    assert out[1] == f"query 0 route 1 weight_bytes {256 * 1536 * 4096 * 2} outputs {8 * 1536}"
    assert out[2].startswith("rejected -1 zero dimension")


@pytest.mark.gpu
def test_plain_c_program_runs_both_routes_on_the_gpu(tmp_path):
    """A plain C program (HIP runtime C API for device memory, no PyTorch)
    runs Direct and Grouped matmul_id on a small bf16 problem: equal bits,
    and within 2e-5 of its own double-precision sum."""
    _need("gcc")
    lib = os.path.join(LIBDIR, "libeidm.so")
    if not os.path.exists(lib):
        pytest.skip("libeidm.so is not built")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "c_abi_gpu"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
                    "-I", os.path.join(rocm, "include"), os.path.join(HERE, "c_abi_gpu.c"), "-L", LIBDIR, "-leidm",
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm", f"-Wl,-rpath,{LIBDIR}",
                    f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", str(exe)], check=True)
    print("[case] plain C program on the GPU", flush=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().splitlines()[-1].startswith("worst ")
