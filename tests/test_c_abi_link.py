"""A plain C program compiles against include/tdm.h and links libtdm.so.

Runs without a GPU: it uses only the host-side calls (cost model, path
queries, status strings) and the validation that precedes any HIP call.
"""
import os
import shutil
import subprocess

import pytest

from tiled_dense_matrix_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "tdm.h"

int main(void) {
  tdm_roofline r;
  if (gemm_roofline(TDM_KIND_F32, 4096, 4096, 4096, &r) != TDM_SUCCESS) return 1;
  if (r.flops != 137438953472.0 || r.bytes != 201326592.0) return 2;
  if (gemm_roofline(TDM_KIND_BF16_F32ACC, 16, 8192, 8192, &r) != TDM_SUCCESS) return 3;
  if (r.bytes != 2.0 * (16.0 * 8192 + 8192.0 * 8192) + 4.0 * 16 * 8192) return 4;
  if (tdm_select_path(TDM_KIND_BF16_F32ACC, 16, 8192, 8192) != TDM_PATH_SKINNY) return 5;
  if (tdm_select_path(TDM_KIND_BF16_F32ACC, 8192, 8192, 8192) != TDM_PATH_MFMA) return 6;
  if (gemm_f32(NULL, NULL, NULL, -1, 1, 1, NULL) != TDM_ERROR_INVALID_VALUE) return 7;
  if (gemm_bf16_f32acc(NULL, NULL, NULL, 0, 5, 5, NULL) != TDM_SUCCESS) return 8;
  if (strcmp(tdm_status_string(TDM_ERROR_NOT_SUPPORTED), "not supported") != 0) return 9;
  if (tdm_version() != TDM_VERSION) return 10;
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_links_and_runs(tmp_path):
    lib = _lib.load()  # builds libtdm.so if it is missing
    del lib
    libdir = os.path.dirname(_lib.LIB_PATH)
    src = tmp_path / "use_tdm.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_tdm"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-ltdm",
                    f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == "ok"
