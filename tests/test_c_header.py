"""The boundary is plain C: include/hattn.h compiles as strict C99, and a C
program links against libhattn.so and gets the validation results and sizes
the header promises (no GPU needed: every call below returns before any
device work)."""
import os
import shutil
import subprocess

import pytest

from compressed_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "hattn.h"

int main(void) {
  size_t sz = 123;
  hattn_decode_plan_t plan = NULL;
  const int32_t pos[2] = {5, 9};
  int fails = 0;
  /* argument errors are reported before anything runs */
  fails += hattn_compress(HATTN_BF16, NULL, 1, 100, 256, NULL, NULL, 8, 4, 0, 1, NULL, NULL) != HATTN_ERR_ARG;
  fails += strlen(hattn_last_error()) == 0;
  fails += hattn_compress(7, NULL, 1, 100, 256, NULL, NULL, 8, 4, 0, 1, NULL, NULL) != HATTN_ERR_ARG;
  /* empty batches are no-ops that need no workspace */
  fails += hattn_compress(HATTN_BF16, NULL, 0, 100, 256, NULL, NULL, 8, 4, 0, 24, NULL, NULL) != HATTN_OK;
  fails += hattn_index_topk(HATTN_BF16, NULL, NULL, NULL, NULL, 0, 4, 16, 128, 1000, 8, NULL, NULL, NULL, &sz,
                            NULL) != HATTN_OK || sz != 0;
  fails += hattn_visible_count(pos, 0, 8, 4, 1023, NULL, NULL) != HATTN_OK;
  /* plan API */
  fails += hattn_decode_plan_create(NULL, &plan) != HATTN_ERR_ARG || plan != NULL;
  fails += hattn_decode_plan_destroy(NULL) != HATTN_OK;
  fails += hattn_decode_desc_size() != (int64_t)sizeof(hattn_decode_desc);
  fails += strcmp(hattn_status_string(HATTN_OK), hattn_status_string(HATTN_ERR_ARG)) == 0;
  printf("abi %d fails %d\n", hattn_abi_version(), fails);
  return fails;
}
"""


@pytest.fixture(scope="module")
def cc():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libhattn.so is not built (run __graft_entry__.build())")
    return gcc


def test_header_is_strict_c99(cc, tmp_path):
    src = tmp_path / "only_header.c"
    src.write_text('#include "hattn.h"\nint hattn_header_compiles(void) { return HATTN_OK; }\n')
    r = subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-c", str(src), "-o", str(tmp_path / "only_header.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_links_and_validates(cc, tmp_path):
    src = tmp_path / "abi_check.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                        "-L", libdir, "-l:libhattn.so", "-Wl,-rpath," + libdir, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "fails 0" in run.stdout
