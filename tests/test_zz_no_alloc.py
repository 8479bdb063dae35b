"""rk_online_softmax_noalloc, the entry point that allocates nothing: its
split partials live in the library's fixed device scratch.  Through the C ABI
it must give rk_online_softmax's results with a caller's workspace, bit for
bit, and the oracle's within tolerance, on consecutive calls that share the
scratch (the second smaller than the first)."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_amd as rk
import rowgen
from tolerance import TOL, rel_err_softmax

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rk.load()
    yield
    torch.cuda.synchronize()


def _check(x, S):
    tol = TOL["f32"] if x.dtype == torch.float32 else TOL["bf16"]
    xd = x.to(DEV)
    y = torch.full_like(xd, float("nan"))
    rk.rk_online_softmax_noalloc(xd, num_splits=S, out=y)
    ref = rk.rk_online_softmax(xd, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), ref.cpu()), S
    err = rel_err_softmax(y, oracle.softmax(x))
    print(f"noalloc {tuple(x.shape)} {x.dtype} S={S} err={err:.3e}", flush=True)
    assert err <= tol


def test_noalloc_consecutive_calls():
    # 64 rows of 262144 at 64 chunks (32 KiB of partials), then a smaller
    # call over the same scratch: 5 odd-length rows at 7 chunks
    _check(rowgen.randn(64, 262144, seed=101, scale=3.0), 64)
    _check(rowgen.randn(5, 40001, seed=103, scale=3.0), 7)


def test_noalloc_auto_bf16_and_limits():
    x = rowgen.randn(16, 100000, seed=107, scale=8.0, dtype=torch.bfloat16)
    assert rk.rk_online_softmax_auto_splits(16, 100000, rk.RK_BF16) > 1
    _check(x, 0)
    _check(rowgen.randn(3, 5000, seed=109), 1)  # one kernel, no scratch
    # M * S = 131072 partials fill the 1 MiB scratch exactly; one more row
    # is refused before anything is enqueued
    _check(rowgen.randn(2048, 4096, seed=113, scale=3.0), 64)
    x = torch.zeros(2049, 4096, device=DEV)
    with pytest.raises(rk.RowKernError) as e:
        rk.rk_online_softmax_noalloc(x, num_splits=64, out=x)
    assert e.value.status == 5
    assert torch.all(x == 0)
