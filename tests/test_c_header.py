"""include/mhc.h as plain C: a C99 program (gcc, -pedantic) that includes
the header, links libmhc.so and calls entry points that return from their
host-side checks (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include "mhc.h"
#include <stdio.h>
int main(void) {
  mhc_params p = {0};
  p.T = 4; p.n = 3; p.d = 64; p.dtype = MHC_BF16; p.t_max = 20; p.eps = 1e-6f;
  mhc_status a = mhc_post(&p, 0, 0, 0, 0, 0);             /* n = 3: unsupported */
  p.n = 4;
  mhc_status b = mhc_post(&p, 0, 0, 0, 0, 0);             /* NULL tensors */
  size_t ws = mhc_pre_workspace_size(&p);
  size_t wq = mhc_workspace_size(&p, MHC_OP_PRE);
  size_t wb = mhc_workspace_size(&p, MHC_OP_PRE_BWD);
  printf("%d %d %d %d %d %d\n", mhc_abi_version(), (int)a, (int)b, ws > 0, wq == ws,
         wb == mhc_pre_bwd_workspace_size(&p) && wb > 0);
  return 0;
}
"""


def test_header_compiles_and_links_as_c(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    import mhc_hyper_connections_amd as m
    if not os.path.exists(m.LIB_PATH):
        from mhc_hyper_connections_amd import build
        build.build(force=False)
    src = tmp_path / "t.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "t"
    libdir = os.path.dirname(m.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-L", libdir, "-lmhc", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.split()
    import re
    ver = int(re.search(r"#define MHC_ABI_VERSION (\d+)", open(os.path.join(ROOT, "include", "mhc.h")).read()).group(1))
    assert out == [str(ver), "5", "1", "1", "1", "1"]
