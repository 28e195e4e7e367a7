"""The boundary from plain C, without a GPU: include/lr_block.h compiles as C99
with gcc, a C program links against liblrblock.so and calls the entry points
that need no device (status strings, workspace sizes, a host-side argument
check), and the dims structs have the same size and field offsets in C as in
the ctypes binding."""
import ctypes
import os
import shutil
import subprocess

import pytest

import rank_bottleneck_amd as rb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(
    not os.path.exists(rb.LIB_PATH) or shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE),
    reason="needs the built library, gcc and the HIP headers")

PROGRAM = r"""
#include <stddef.h>
#include <stdio.h>
#include "lr_block.h"
int main(void) {
  lr_dims d = {16384, 4096, 1024, 3, 0, 1e-6f, LR_BF16, LR_ACT_SILU};
  lr_mlp_dims m = {16384, 4096, 11008, 1024, 1e-6f, LR_BF16};
  printf("%s\n", lr_status_str(LR_EWORKSPACE));
  printf("%zu %zu %zu %zu\n", lr_block_workspace_size(&d, 0), lr_block_workspace_size(&d, 1),
         lr_mlp_workspace_size(&m, 0), lr_mlp_workspace_size(&m, 1));
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(lr_dims), offsetof(lr_dims, T), offsetof(lr_dims, d),
         offsetof(lr_dims, r), offsetof(lr_dims, g), offsetof(lr_dims, d_norm), offsetof(lr_dims, eps),
         offsetof(lr_dims, dtype), offsetof(lr_dims, act));
  printf("%zu %zu %zu %zu %zu %zu %zu\n", sizeof(lr_mlp_dims), offsetof(lr_mlp_dims, T), offsetof(lr_mlp_dims, d),
         offsetof(lr_mlp_dims, f), offsetof(lr_mlp_dims, r), offsetof(lr_mlp_dims, eps),
         offsetof(lr_mlp_dims, dtype));
  /* rejected on the host (null x with T > 0): nothing is launched */
  printf("%d\n", (int)lr_block_fwd(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(rb.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE, str(src), "-L", libdir, "-llrblock",
           f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.split("\n")
    assert out[0] == "LR_EWORKSPACE"
    # the same sizes as the binding reports
    d = rb.make_dims(16384, 4096, 1024, 3, "silu", "bf16")
    m = rb.make_mlp_dims(16384, 4096, 11008, 1024, "bf16")
    assert [int(v) for v in out[1].split()] == [rb.lr_block_workspace_size(d, False), rb.lr_block_workspace_size(d, True),
                                                rb.lr_mlp_workspace_size(m, False), rb.lr_mlp_workspace_size(m, True)]
    # struct layouts match the ctypes mirrors field by field
    c_dims = [int(v) for v in out[2].split()]
    py_dims = [ctypes.sizeof(rb.LrDims)] + [getattr(rb.LrDims, f).offset
                                            for f in ("T", "d", "r", "g", "d_norm", "eps", "dtype", "act")]
    assert c_dims == py_dims
    c_mlp = [int(v) for v in out[3].split()]
    py_mlp = [ctypes.sizeof(rb.LrMlpDims)] + [getattr(rb.LrMlpDims, f).offset
                                              for f in ("T", "d", "f", "r", "eps", "dtype")]
    assert c_mlp == py_mlp
    assert int(out[4]) == rb.LR_EINVAL
