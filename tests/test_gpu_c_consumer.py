"""The boundary from plain C on the GPU: a C99 program that uses only
include/mdc.h and the HIP runtime's C API (no torch, no C++) dispatches for
every rank, combines for every rank and checks the identity round trip
(identity expert, weights 0.5 + 0.5: out = x bit for bit) and the counts."""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_route_histogram_amd as mdc  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

C_SRC = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>
#include "mdc.h"

#define HIPCHK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); return 2; } } while (0)
#define MDCCHK(x) do { mdc_status s_ = (x); if (s_ != MDC_OK) { \
    fprintf(stderr, "mdc error %s at line %d\n", mdc_status_string(s_), __LINE__); return 3; } } while (0)

enum { W = 2, BS = 64, H = 256, K = 2, E = 4, L = E / W };

/* bf16 of a small integer (exact for |v| <= 256) */
static uint16_t bf16_of_int(int v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

int main(void) {
    const int64_t A = (int64_t)W * BS * (L < K ? L : K);
    mdc_shape sh;
    size_t wsb = 0;
    int s, t, h, k, j, r;
    void *x, *ids, *row_idx, *scales, *out;
    void *ex[W], *as[W], *rc[W], *tn[W], *ws[W];
    uint16_t* hx = malloc((size_t)W * BS * H * 2);
    uint16_t* hout = malloc((size_t)BS * H * 2);
    int32_t* hids = malloc((size_t)W * BS * K * 4);
    float* hsc = malloc((size_t)BS * K * 4);
    int64_t total = 0;

    memset(&sh, 0, sizeof sh);
    sh.world = W; sh.bs = BS; sh.hidden = H; sh.topk = K; sh.num_experts = E; sh.capacity = A;
    for (s = 0; s < W; ++s)
        for (t = 0; t < BS; ++t) {
            for (h = 0; h < H; ++h)
                hx[((size_t)s * BS + t) * H + h] = bf16_of_int(((s * BS + t) * 7 + h) % 255 - 127);
            for (k = 0; k < K; ++k) hids[((size_t)s * BS + t) * K + k] = (s + t + k) % E;   /* distinct */
        }
    for (t = 0; t < BS * K; ++t) hsc[t] = 0.5f;

    HIPCHK(hipMalloc(&x, (size_t)W * BS * H * 2));
    HIPCHK(hipMalloc(&ids, (size_t)W * BS * K * 4));
    HIPCHK(hipMalloc(&row_idx, (size_t)W * BS * K * 4));
    HIPCHK(hipMalloc(&scales, (size_t)BS * K * 4));
    HIPCHK(hipMalloc(&out, (size_t)BS * H * 2));
    HIPCHK(hipMemcpy(x, hx, (size_t)W * BS * H * 2, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(ids, hids, (size_t)W * BS * K * 4, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(scales, hsc, (size_t)BS * K * 4, hipMemcpyHostToDevice));
    MDCCHK(mdc_dispatch_workspace(&sh, &wsb));
    for (j = 0; j < W; ++j) {
        HIPCHK(hipMalloc(&ex[j], (size_t)A * H * 2));
        HIPCHK(hipMalloc(&as[j], (size_t)A * 3 * 4));
        HIPCHK(hipMalloc(&rc[j], (size_t)L * W * 4));
        HIPCHK(hipMalloc(&tn[j], (size_t)L * 8));
        HIPCHK(hipMalloc(&ws[j], wsb));
    }

    /* the dispatch of every destination rank, on the null stream */
    for (j = 0; j < W; ++j) {
        sh.rank = j;
        MDCCHK(mdc_dispatch(&sh, x, (const int32_t*)ids, NULL, NULL, ex[j], (int32_t*)as[j], (int32_t*)rc[j],
                            (int64_t*)tn[j], (int32_t*)row_idx, NULL, ws[j], wsb, NULL));
    }
    HIPCHK(hipDeviceSynchronize());
    for (j = 0; j < W; ++j) {
        int64_t n[L];
        int32_t last;
        HIPCHK(hipMemcpy(n, tn[j], sizeof n, hipMemcpyDeviceToHost));
        HIPCHK(hipMemcpy(&last, (int32_t*)rc[j] + L * W - 1, 4, hipMemcpyDeviceToHost));
        for (k = 0; k < L; ++k) total += n[k];
        if (last != (int32_t)(n[0] + n[1])) { fprintf(stderr, "rank %d: counts disagree\n", j); return 4; }
    }
    if (total != (int64_t)W * BS * K) { fprintf(stderr, "received %lld routes\n", (long long)total); return 5; }

    /* the combine of every source rank: identity expert, 0.5 x + 0.5 x = x */
    for (r = 0; r < W; ++r) {
        sh.rank = r;
        MDCCHK(mdc_combine(&sh, (const void* const*)ex, (const int32_t* const*)as, (const int32_t* const*)rc,
                           (const int32_t*)row_idx + (size_t)r * BS * K, (const int32_t*)ids + (size_t)r * BS * K,
                           (const float*)scales, NULL, NULL, NULL, NULL, NULL, out, NULL, 0, NULL));
        HIPCHK(hipMemcpy(hout, out, (size_t)BS * H * 2, hipMemcpyDeviceToHost));
        if (memcmp(hout, hx + (size_t)r * BS * H, (size_t)BS * H * 2) != 0) {
            fprintf(stderr, "rank %d: round trip differs\n", r);
            return 6;
        }
    }
    printf("ok %lld\n", (long long)total);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_program_round_trip_on_the_gpu(tmp_path):
    src = tmp_path / "roundtrip.c"
    src.write_text(C_SRC)
    exe = tmp_path / "roundtrip"
    libdir = os.path.dirname(mdc.LIB_PATH)
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), str(src),
                         "-o", str(exe), "-L", libdir, "-l:libmdc.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                         f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    print("running the C round trip", flush=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stderr)
    assert run.stdout.split() == ["ok", str(2 * 64 * 2)]
