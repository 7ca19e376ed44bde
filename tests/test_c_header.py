"""The ABI header is plain C: a C99 program that includes it compiles
without warnings, links against the library and gets the same host-side
answers (parameter count, path, workspace sizes, status text) as the Python
binding.  No GPU is touched."""
import os
import shutil
import subprocess

import pytest

from test_learned_neural_amd import titans_mem as tmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "titans_mem.h"

int main(void) {
  titans_mem_desc d;
  memset(&d, 0, sizeof d);
  d.abi_version = TITANS_MEM_ABI_VERSION;
  d.B = 8; d.H = 16; d.N = 16384; d.d = 64; d.hidden = 256; d.n_layers = 2;
  d.activation = TM_ACT_SILU; d.io_dtype = TM_IO_BF16; d.read_mode = TM_READ_AFTER_WRITE; d.flags = 0u;
  printf("%d %lld %d %lld %lld %s\n", (int)titans_mem_abi_version(), (long long)titans_mem_param_count(&d),
         (int)titans_mem_select_path(&d, 64), (long long)titans_mem_workspace_bytes(&d, 64),
         (long long)titans_mem_backward_workspace_bytes(&d, 64), titans_mem_status_string(TM_OK));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c99_and_links(tmp_path):
    lib = tmm.load()   # builds nothing; fails if the library is missing
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(tmm.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-ltitans_mem", "-Wl,-rpath," + libdir],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=120).stdout.split()
    desc = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16")
    assert int(out[0]) == lib.titans_mem_abi_version()
    assert int(out[1]) == tmm.param_count(desc) == 2 * 64 * 256
    assert int(out[2]) == tmm.select_path(desc, 64)
    assert int(out[3]) == tmm.workspace_bytes(desc, 64)
    assert int(out[4]) == tmm.backward_workspace_bytes(desc, 64)
    assert out[5].lower().startswith("ok")
