"""The boundary is a plain C ABI: include/moe_finalize.h compiles as strict C99, and a C program
links against libmoe_finalize.so and calls its host-only entry points (no GPU involved)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "moe_expert_output_amd", "lib")

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "moe_finalize.h"

int main(void) {
    /* host-only helpers: sizes, error strings, version */
    if (moe_finalize_sf_size(64, 6144, MOE_SF_SWIZZLED_128x4) != (size_t)128 * 384) return 1;
    if (moe_finalize_sf_size(5, 48, MOE_SF_LINEAR) != 15) return 2;
    if (moe_finalize_workspace_size(128, 7168, 8) != 256 + 128 * 128) return 3;
    if (strcmp(moe_finalize_error_string(MOE_FIN_OK), "success") != 0) return 4;
    if (moe_finalize_version() < 100) return 5;
    /* validation happens before anything touches a device: a bad top_k, a bad hidden, T = 0 */
    if (moe_finalize_run(NULL, 0, NULL, NULL, MOE_DTYPE_FP32, NULL, 1.0f, NULL, 4, 1024, 0,
                         MOE_DTYPE_BF16, NULL) != MOE_FIN_ERR_BAD_TOPK) return 6;
    if (moe_finalize_rmsnorm_run(NULL, 0, NULL, NULL, MOE_DTYPE_FP32, NULL, 1.0f, NULL, NULL,
                                 1e-6f, NULL, NULL, NULL, 0, 4, 1020, 8, MOE_DTYPE_BF16,
                                 NULL) != MOE_FIN_ERR_HIDDEN) return 7;
    if (moe_rank_sum_rmsnorm_run(NULL, 4, NULL, NULL, 1e-6f, NULL, NULL, NULL, 0, 0, 1024,
                                 MOE_DTYPE_BF16, NULL) != MOE_FIN_OK) return 8;
    printf("c abi ok\n");
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_is_c99_and_a_c_program_links(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", LIB_DIR, "-lmoe_finalize", f"-Wl,-rpath,{LIB_DIR}",
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c abi ok" in r.stdout, (r.returncode, r.stdout, r.stderr)
