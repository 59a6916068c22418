"""A plain C99 program builds against include/mdc.h alone, links libmdc.so
and gets the same answers from the host-side calls as the Python binding
(no GPU needed: the calls it makes return before anything is enqueued).
This checks that the boundary needs no C++ and no torch."""
import os
import shutil
import subprocess

import pytest

import combine_route_histogram_amd as mdc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "mdc.h"

int main(void) {
    mdc_shape sh;
    size_t dws = 0, cws = 0, fws = 0;
    memset(&sh, 0, sizeof sh);
    sh.world = 8; sh.rank = 0; sh.bs = 2048; sh.hidden = 7168; sh.topk = 8;
    sh.num_experts = 128; sh.capacity = 131072;
    if (mdc_abi_version() != MDC_ABI_VERSION) return 10;
    if (mdc_dispatch_workspace(&sh, &dws) != MDC_OK || dws == 0) return 11;
    if (mdc_combine_workspace(&sh, &cws) != MDC_OK) return 12;
    if (mdc_ffn_workspace(&sh, 4096, &fws) != MDC_OK || fws == 0) return 13;
    /* null tensors are refused before anything is enqueued */
    if (mdc_dispatch(&sh, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                     NULL, 0, NULL) != MDC_ERR_NULLPTR) return 14;
    if (mdc_dispatch_workspace(NULL, &dws) != MDC_ERR_NULLPTR) return 15;
    /* a shape outside the supported range */
    sh.topk = MDC_MAX_TOPK + 1;
    if (mdc_dispatch_workspace(&sh, &dws) != MDC_ERR_UNSUPPORTED) return 16;
    printf("%d %zu %zu %zu %s\n", mdc_abi_version(), dws, cws, fws, mdc_status_string(MDC_ERR_NULLPTR));
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_program_uses_the_boundary(tmp_path):
    src = tmp_path / "consumer.c"
    src.write_text(C_SRC)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(mdc.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-l:libmdc.so", f"-Wl,-rpath,{libdir}"],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stderr)
    ver, dws, cws, fws, name = out.stdout.strip().split(maxsplit=4)
    share = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=131072)
    assert int(ver) == mdc.mdc_abi_version()
    assert int(dws) == mdc.mdc_dispatch_workspace(share)
    assert int(cws) == mdc.mdc_combine_workspace(share)
    assert int(fws) == mdc.mdc_ffn_workspace(share, 4096)
    assert name == mdc.mdc_status_string(1)
