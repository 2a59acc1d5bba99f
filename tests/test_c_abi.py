"""The boundary is a plain C ABI: a C99 program that includes only
include/uniprefill.h (plus HIP's runtime API header for hipStream_t) compiles
with gcc, links libuniprefill.so and calls it (host-side helpers and
argument checks only, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

import token_block_sparsification_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include "uniprefill.h"

int main(void) {
  int32_t cu[4] = {0, 100, 100, 300};
  int32_t cb[4];
  int64_t n = 0;
  up_status st = up_make_cu_blocks(3, cu, 64, cb, &n);
  if (st != UP_OK || n != 6 || cb[0] != 0 || cb[1] != 2 || cb[2] != 2 || cb[3] != 6) return 1;
  size_t ws = 0;
  if (up_compact_workspace_size(3, cu, 64, &ws) != UP_OK || ws == 0 || ws % 256) return 2;
  st = up_score(1, cu, NULL, NULL, NULL, 0, 0, 4, NULL, 0, 0, 2, 96, 128, 64, 0.f, NULL, NULL,
                NULL, 0, NULL);
  if (st != UP_ERR_UNSUPPORTED) return 3;
  printf("%d %s|%s\n", up_abi_version(), up_status_string(st), up_last_error());
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c_and_links(tmp_path):
    lib = U.lib()._name
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(lib)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           str(src), "-L", libdir, "-l:" + os.path.basename(lib), "-Wl,-rpath," + libdir, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    ver, rest = out.stdout.strip().split(" ", 1)
    assert int(ver) == U.up_abi_version()
    status, msg = rest.split("|", 1)
    assert status == "UP_ERR_UNSUPPORTED" and "head_dim" in msg
