"""The boundary from C: include/rowkern.h and include/rowkern_tune.h compile
as C99 with gcc (-Wall -Wextra -Werror), a C program links against
librowkern.so, takes the address of every entry point the headers declare,
and calls only paths that return before any HIP call (version, status
strings, sizes, rejected arguments, M = 0).  No GPU is needed."""
import os
import shutil
import subprocess

import pytest

import row_wise_amd as rk
from test_abi import ROOT, declared_symbols

PROGRAM = r"""
#include "rowkern.h"
#include "rowkern_tune.h"
#include <stdint.h>
#include <stdio.h>

typedef void (*any_fn)(void);
#define CHECK(c) do { if (!(c)) { printf("failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void)
{
    /* every declared entry point resolves */
    const any_fn table[] = { %(TABLE)s };
    for (size_t i = 0; i < sizeof table / sizeof table[0]; ++i)
        CHECK(table[i] != 0);

    CHECK(rk_version() == RK_VERSION);
    for (int s = RK_OK; s <= RK_ERR_SCRATCH; ++s)
        CHECK(rk_status_string((rk_status)s) != 0);

    /* fake, 16-byte aligned device addresses: never dereferenced */
    const void *x = (const void *)(uintptr_t)0x100000;
    void *y = (void *)(uintptr_t)0x900000;

    CHECK(rk_softmax(0, 0, 0, 8, 8, 8, RK_F32, 0) == RK_OK);
    CHECK(rk_softmax(x, y, 4, 0, 8, 8, RK_F32, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_softmax(x, y, 4, 8, 7, 8, RK_F32, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_online_softmax(x, y, 4, 4096, 4096, 4096, RK_F32, 64, 0, 0, 0) == RK_ERR_WORKSPACE);
    CHECK(rk_online_softmax_workspace_bytes(64, 262144, 64, RK_F32) == (size_t)64 * 64 * 8);
    CHECK(rk_online_softmax_auto_splits(16384, 4096, RK_F32) == 1);
    CHECK(rk_layernorm_gelu(x, 0, 0, y, 4, 8, 8, 8, 1e-5f, RK_BF16, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_layernorm_gelu_ex(x, x, x, y, 4, 8, 8, 8, 1e-5f, RK_F32, (rk_gelu_kind)3, 1, 0, 0,
                               0) == RK_ERR_INVALID_ARG);
    CHECK(rk_gelu(x, y, 4, 8, 8, 8, RK_F32, RK_GELU_NONE, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_layernorm_gelu_workspace_bytes(64, 262144, 64, RK_F32) == (size_t)64 * 65 * 8);
    CHECK(rk_rmsnorm(x, x, y, 4, 8, 8, 8, 0.0f, RK_F32, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_row_sum(x, y, -1, 8, 8, RK_F32, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_row_sum_ex(x, y, 4, 4096, 4096, RK_F32, 8, 0, 0, 0) == RK_ERR_WORKSPACE);
    CHECK(rk_row_max_ex(x, y, 4, 4096, 4096, RK_F32, -1, 0, 0, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_row_reduce_workspace_bytes(64, 262144, 32, RK_F32) == (size_t)64 * 32 * 4);
    CHECK(rk_gelu(x, y, 4, 8, 8, 8, RK_F32, (rk_gelu_kind)7, 0) == RK_ERR_INVALID_ARG);
    CHECK(rk_flash_attention(x, x, x, y, 0, 32, 1024, 128, 0, 0, 0, 0, 0.1f, 0, RK_BF16, 0) ==
          RK_OK);
    CHECK(rk_flash_attention(x, x, x, y, 1, 1, 64, 0, 0, 0, 0, 0, 0.1f, 0, RK_BF16, 0) ==
          RK_ERR_INVALID_ARG);
    /* partials beyond the fixed scratch (x and y 256 MiB apart: no overlap) */
    CHECK(rk_online_softmax_noalloc((const void *)(uintptr_t)0x10000000,
                                    (void *)(uintptr_t)0x20000000, 2049, 4096, 4096, 4096,
                                    RK_F32, 64, 0) == RK_ERR_SCRATCH);
    CHECK(rk__variant_count(RK_OP_SOFTMAX, RK_F32) > 0);
    printf("c abi ok\n");
    return 0;
}
"""


def test_headers_compile_and_link_from_c(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    rk.load()  # the library exists (built)
    names = declared_symbols()
    src = PROGRAM.replace("%(TABLE)s", ", ".join(f"(any_fn){n}" for n in names))
    c = tmp_path / "abi.c"
    c.write_text(src)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(rk.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(c),
           "-L", libdir, "-lrowkern", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and "c abi ok" in run.stdout, run.stdout + run.stderr
