"""The largest problems the entry points accept, against the oracle.

The longest row is N = 2^30 elements (4 GiB in fp32): every form of the
softmax and of the row sum and max (one workgroup per row, and split) take
it as one row, and the oracle's statistics of the whole row check 2304
sampled outputs (the first and last 128 columns and 2048 seeded others;
"Triton Kernel 实现练习" §2.4, §2.5).  A
2^28-column bf16 LayerNorm+GeLU row is checked whole.  The tallest grid a
register tile takes is 2^26 - 4 rows of 8 (one wave per row, four rows per
workgroup, 2^32 - 256 work-items); one more workgroup's rows are refused
with RK_ERR_UNSUPPORTED before anything is launched.

Inputs are drawn on the GPU from a seeded generator and copied to the host
for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_amd as rk
from tolerance import TOL, rel_err_floor1, rel_err_softmax

pytestmark = pytest.mark.gpu
DEV = "cuda"
EPS = float(np.float32(1e-5))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rk.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(msg):
    print(msg, flush=True)


def draw(shape, seed, scale=1.0, dtype=torch.float32):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(dtype)


def sample_columns(N, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(128, N - 128), 2048, replace=False)
    return np.unique(np.concatenate([np.arange(128), np.arange(N - 128, N), mid]))


def test_longest_row_softmax_forms():
    N = 1 << 30
    xd = draw((1, N), 601, scale=3.0)
    x = xd.cpu()
    say("longest row: oracle statistics of 2^30 values")
    m, d = oracle.softmax_stats(x[0])
    cols = sample_columns(N, 601)
    ref = oracle.softmax_apply(x[0, cols].double().numpy(), m, d)
    idx = torch.from_numpy(cols).to(DEV)
    forms = {
        "rk_softmax": lambda: rk.rk_softmax(xd),
        "online S=1": lambda: rk.rk_online_softmax(xd, num_splits=1),
        "online auto (workspace)": lambda: rk.rk_online_softmax(xd, num_splits=0),
        "online auto (no alloc)": lambda: rk.rk_online_softmax_noalloc(xd, num_splits=0),
    }
    for name, run in forms.items():
        y = run()
        err = rel_err_softmax(y[0, idx].cpu(), ref)
        say(f"longest row {name}: err {err:.3e}")
        assert err <= TOL["f32"], name
        del y
        torch.cuda.empty_cache()


def test_longest_row_sum_and_max():
    N = 1 << 30
    xd = draw((1, N), 603)
    x = xd.cpu()
    s = rk.rk_row_sum(xd).cpu().double().numpy()
    mx = rk.rk_row_max(xd).cpu()
    # the split forms (auto: 2048 chunks of 2^19)
    assert rk.rk_row_reduce_auto_splits(1, N, rk.RK_F32) == 2048
    s_split = rk.rk_row_sum_ex(xd).cpu().double().numpy()
    mx_split = rk.rk_row_max_ex(xd).cpu()
    say("longest row: oracle sum and max of 2^30 values")
    xn = x.double().numpy()
    ref_s = oracle.row_sum(xn)
    ref_m = oracle.row_max(xn)
    scale = np.abs(xn).sum()
    assert abs(s[0] - ref_s[0]) / scale <= TOL["f32"]
    assert abs(s_split[0] - ref_s[0]) / scale <= TOL["f32"]
    assert mx[0].item() == ref_m[0] and mx_split[0].item() == ref_m[0]


def test_long_bf16_layernorm_row():
    N = 1 << 28
    xd = draw((1, N), 605, dtype=torch.bfloat16)
    g = torch.Generator(device=DEV).manual_seed(606)
    wd = (1.0 + 0.1 * torch.randn(N, generator=g, device=DEV)).to(torch.bfloat16)
    bd = (0.1 * torch.randn(N, generator=g, device=DEV)).to(torch.bfloat16)
    y = rk.rk_layernorm_gelu(xd, wd, bd, EPS).cpu()
    say("long bf16 row: oracle LayerNorm+GeLU of 2^28 values")
    ref = oracle.layernorm_gelu(xd.cpu(), wd.cpu(), bd.cpu(), EPS)
    err = rel_err_floor1(y, ref)
    say(f"long bf16 row LayerNorm+GeLU: err {err:.3e}")
    assert err <= TOL["bf16"]


def test_tallest_tile_grid():
    M, N = (1 << 26) - 4, 8
    xd = draw((M, N), 607, scale=4.0)
    wd = 1.0 + 0.1 * draw((N,), 608)
    bd = 0.1 * draw((N,), 609)
    x = xd.cpu()
    y = rk.rk_softmax(xd).cpu()
    say("tallest grid: oracle softmax of 2^26 - 4 rows")
    err = rel_err_softmax(y, oracle.softmax(x))
    assert err <= TOL["f32"], err
    del y
    z = rk.rk_layernorm_gelu(xd, wd, bd, EPS).cpu()
    say("tallest grid: oracle LayerNorm+GeLU of 2^26 - 4 rows")
    err = rel_err_floor1(z, oracle.layernorm_gelu(x, wd.cpu(), bd.cpu(), EPS))
    assert err <= TOL["f32"], err
    # four more rows would need 2^32 work-items: refused before any launch
    lib = rk.load()
    big = torch.empty(1 << 26, N, device=DEV)
    st = lib.rk_softmax(big.data_ptr(), big.data_ptr(), 1 << 26, N, N, N, rk.RK_F32,
                        torch.cuda.current_stream().cuda_stream)
    assert st == 2
