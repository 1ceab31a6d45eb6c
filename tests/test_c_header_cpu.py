"""The C ABI from plain C: include/vbm.h compiles as C99 with warnings as errors,
and a C program linked against libvbm.so builds a grid on the host (vbm_build needs
no GPU), reads its header, frees the blob, and gets the documented error codes."""
import os
import subprocess

import pytest

from nanovdb_stencil_filtering_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include "vbm.h"

int main(void) {
  /* a 2 x 2 x 2 cube at the origin and one voxel in the next leaf along x */
  int32_t ijk[9 * 3];
  int n = 0;
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 2; ++y)
      for (int z = 0; z < 2; ++z) { ijk[3 * n] = x; ijk[3 * n + 1] = y; ijk[3 * n + 2] = z; ++n; }
  ijk[3 * n] = 8; ijk[3 * n + 1] = 0; ijk[3 * n + 2] = 0; ++n;
  vbm_grid grid;
  void* blob = NULL;
  int rc = vbm_build(ijk, n, 7, &grid, &blob);
  if (rc != VBM_OK || !blob) { printf("build failed %d %s\n", rc, vbm_strerror(rc)); return 1; }
  printf("n_active=%llu n_leaves=%u n_blocks=%u blob_bytes=%llu\n", (unsigned long long)grid.n_active,
         grid.n_leaves, grid.n_blocks, (unsigned long long)grid.blob_bytes);
  vbm_free_blob(blob);
  int32_t far_away[3] = {0, 0, 1 << 30};
  rc = vbm_build(far_away, 1, 7, &grid, &blob);
  printf("range=%d blob_null=%d\n", rc, blob == NULL);
  rc = vbm_build(ijk, n, 5, &grid, &blob);
  printf("width=%d\n", rc);
  printf("arg=%s\n", vbm_strerror(VBM_ERR_ARG));
  return 0;
}
"""


def test_c_program_against_the_header(tmp_path):
    lib = B.LIB
    if not os.path.exists(lib):
        pytest.skip("libvbm.so is not built")
    src = tmp_path / "use_vbm.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_vbm"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", os.path.dirname(lib), "-lvbm",
                    "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    lines = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines()
    assert lines[0].startswith("n_active=9 n_leaves=2 n_blocks=1 "), lines
    assert lines[1:] == ["range=-5 blob_null=1", "width=-1", "arg=invalid argument"], lines
