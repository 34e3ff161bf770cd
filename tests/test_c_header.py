"""The boundary is plain C: include/fa.h compiles as C99 with gcc (-Wall
-Werror -pedantic), and a C program links libfa.so and calls through it. The
calls made here all fail argument validation before any device work, so the
test needs no GPU."""
import os
import shutil
import subprocess

import pytest

from attention_forward_online_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "fa.h"

int main(void) {
  /* every declared entry point is callable from C */
  const long long st[3] = {0, 128, 100};   /* row stride < D: a stride error */
  char* a = (char*)0x10000;
  int bad = 0;
  if (fa_fwd(a, a, a, a, (float*)a, 1, 4, 3, 64, 64, 128, 0.125f, 1, 0, FA_BF16, NULL) != FA_ERR_GQA) bad |= 1;
  if (fa_fwd_ex(a, a, a, a, (float*)a, 1, 4, 2, 64, 64, 40, 0.125f, 1, 0, FA_F16, 0, NULL) != FA_ERR_HEAD_DIM) bad |= 2;
  if (fa_fwd_strided(a, a, a, a, (float*)a, 1, 4, 2, 64, 64, 128, st, NULL, NULL, NULL,
                     0.125f, 1, 0, FA_BF16, 0, NULL) != FA_ERR_STRIDE) bad |= 4;
  if (fa_fwd_block_sparse(a, a, a, a, (float*)a, 1, 4, 2, 64, 64, 128, (const unsigned char*)a,
                          1, 3, 0.125f, 0, 0, FA_F32, 0, NULL) != FA_ERR_MASK) bad |= 8;
  if (fa_bwd(a, a, a, a, a, (const float*)a, (float*)a, (float*)a, (float*)a, 0, 4, 2, 64, 64, 128,
             0.125f, 1, 0, FA_BF16, NULL) != FA_ERR_SHAPE) bad |= 16;
  if (fa_plan_splits(1, 4, 3, 64, 64, 128, 0, 0, FA_BF16) != -FA_ERR_GQA) bad |= 32;
  if (fa_schedule_table(1, 4, 4, 256, 256, 64, 1, 0, FA_F32, 8, NULL, 0, NULL) <= 8) bad |= 64;
  if (strcmp(fa_status_string(FA_OK), "ok") != 0) bad |= 128;
  printf("%d %d %d\n", bad, FA_MAX_SPLITS, FA_MASK_BLOCK_Q * FA_MASK_BLOCK_K);
  return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_c99_and_library_links_from_c(tmp_path):
    lib = _lib.library_path()
    _lib.lib()                                   # builds it if needed
    src = tmp_path / "use_fa.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "use_fa"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), lib, f"-Wl,-rpath,{os.path.dirname(lib)}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert r.stdout.split() == ["0", str(_lib.FA_MAX_SPLITS), str(128 * 64)]
