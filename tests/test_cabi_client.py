"""The library from a plain C program: tests/abi_client.c is compiled with gcc
as strict C99 against include/gemm355.h and linked to libgemm355.so and the
system HIP runtime, with no Python or PyTorch in the process that runs it.

* CPU: the header is valid C99 and the client compiles and links without a
  warning (every symbol it calls is exported);
* GPU: the client's products (automatic plan, forced split-K, persistent
  grid, E4M3 with bf16 output and a caller workspace, a scaled batch through
  the allocation-free entry point, a convolution with padding, stride and
  dilation, the quantiser on tensors whose scale is exactly 1, K = 0, an
  argument error) equal its exact reference bit for bit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "dense_tiled_gemm_fp8_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def compile_client(out_dir):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not on PATH")
    exe = os.path.join(str(out_dir), "abi_client")
    cmd = [gcc, "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_client.c"), "-o", exe,
           "-L" + LIBDIR, "-lgemm355", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout + r.stderr
    return exe


def test_client_compiles_as_c99(tmp_path):
    exe = compile_client(tmp_path)
    assert os.path.getsize(exe) > 0


@pytest.mark.gpu
def test_client_products_exact(tmp_path):
    exe = compile_client(tmp_path)
    print("abi_client: running", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0 and "all cases ok" in r.stdout, r.stdout + r.stderr
    for case in ("gemm_bf16_auto", "gemm_bf16_split4", "gemm_bf16_persistent", "plan",
                 "gemm_ex_e4m3_bf16", "gemm_noalloc_batch_0", "gemm_noalloc_batch_1", "conv_auto",
                 "conv_split3", "quantize_f32_e4m3", "quantize_bf16_e4m3", "quantize_f32_e5m2",
                 "quantize_bf16_e5m2", "gemm_k0"):
        assert "case %s ok" % case in r.stdout, case
