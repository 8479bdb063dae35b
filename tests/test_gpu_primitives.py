"""Parity of the standalone primitives with the CPU oracle: rk_row_sum,
rk_row_max ("Triton Kernel 实现练习" §2.2, §2.3) and the elementwise rk_gelu
(§3.4).  Row sums: error relative to sum |x| of the row, 1e-5 fp32 / 1e-2
bf16; row max: bit-exact; GeLU: relative error with the denominator floored
at 1."""
import math

import numpy as np
import pytest
import torch

import oracle
import row_wise_amd as rk
import rowgen
from tolerance import TOL, rel_err_floor1, rel_err_sum

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTYPES = [torch.float32, torch.bfloat16]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rk.load()
    yield
    torch.cuda.synchronize()


def key(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


def tol_of(dtype):
    return TOL[key(dtype)]


def say(msg):
    print(msg, flush=True)


def check_reductions(x, xd, dtype, what=""):
    s = rk.rk_row_sum(xd)
    err = rel_err_sum(s, oracle.row_sum(x), x.double().numpy())
    assert err <= tol_of(dtype), (what, "sum", err)
    m = rk.rk_row_max(xd).cpu().double().numpy()
    assert np.array_equal(m, oracle.row_max(x), equal_nan=True), (what, "max")
    return err


@pytest.mark.parametrize("name", ["ln_gelu_f32_4096x768", "softmax_f32_8192x1000",
                                  "online_f32_64x262144", "bf16_16384x4096"])
def test_workloads(name):
    d = rowgen.make(name)
    x = d["x_softmax"]
    err = check_reductions(x, x.to(DEV), x.dtype, name)
    say(f"row_sum {name} err={err:.3e}")


EDGE_N = [1, 2, 3, 63, 64, 65, 767, 1000, 1025, 4095, 4097, 16385, 32769, 40000, 262147]


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_shapes(dtype, N):
    for M in (1, 257) if N < 100000 else (1, 5):
        say(f"reduce {key(dtype)} M={M} N={N}")
        x = rowgen.randn(M, N, seed=M * 11 + N, scale=3.0, dtype=dtype)
        x[::3] += 7.0
        check_reductions(x, x.to(DEV), dtype, (M, N))


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_pitch_and_misaligned(dtype):
    M, N, ld = 37, 3001, 3072
    xb = rowgen.randn(M, ld, seed=97, dtype=dtype)
    check_reductions(xb[:, :N], xb.to(DEV)[:, :N], dtype, "pitch")
    flat = rowgen.randn(1, M * N + 1, seed=98, dtype=dtype)[0]
    check_reductions(flat[1:].view(M, N), flat.to(DEV)[1:].view(M, N), dtype, "misaligned")


def test_special_rows():
    x = rowgen.randn(6, 5000, seed=99)
    x[0, 17] = math.nan
    x[1, :] = -math.inf
    x[2, 4999] = math.inf
    x[3, :] = 0.0
    x[4, :2500] = 0.5
    x[4, 2500:] = -0.5  # exact cancellation
    m = rk.rk_row_max(x.to(DEV)).cpu().numpy()
    assert np.isnan(m[0]) and m[1] == -np.inf and m[2] == np.inf and m[3] == 0.0
    s = rk.rk_row_sum(x.to(DEV)).cpu().numpy()
    assert np.isnan(s[0]) and s[1] == -np.inf and s[2] == np.inf
    assert s[3] == 0.0 and s[4] == 0.0
    ref = oracle.row_sum(x[5:])
    assert abs(s[5] - ref[0]) <= 1e-5 * x[5].abs().sum().item()


def test_sum_deterministic_and_empty():
    x = rowgen.randn(64, 262144, seed=101).to(DEV)
    a, b = rk.rk_row_sum(x), rk.rk_row_sum(x)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    e = torch.empty(0, 10, device=DEV)
    assert rk.rk_row_sum(e).shape == (0,) and rk.rk_row_max(e).shape == (0,)


# ------------------------------------------- split row sum and max (_ex)


def check_split(x, xd, dtype, S, what=""):
    """rk_row_sum_ex / rk_row_max_ex at split count S against the oracle:
    the sum within the tolerance of sum |x|, the max bit-exact and equal to
    rk_row_max (max is exact whatever the order)."""
    s = rk.rk_row_sum_ex(xd, num_splits=S)
    err = rel_err_sum(s, oracle.row_sum(x), x.double().numpy())
    assert err <= tol_of(dtype), (what, S, "sum", err)
    m = rk.rk_row_max_ex(xd, num_splits=S)
    assert np.array_equal(m.cpu().double().numpy(), oracle.row_max(x), equal_nan=True), \
        (what, S, "max")
    return err


SPLIT_N = [1, 5, 1000, 4099, 65536, 262147]


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("N", SPLIT_N)
def test_split_shapes(dtype, N):
    """Every split count from 1 to past the vector count (empty chunks),
    ragged N, rows offset by +7 every third row."""
    for M in (1, 3, 70):
        x = rowgen.randn(M, N, seed=5 * M + N, scale=3.0, dtype=dtype)
        x[::3] += 7.0
        xd = x.to(DEV)
        for S in (0, 1, 2, 3, 7, 64, 1000):
            check_split(x, xd, dtype, S, (M, N))
    say(f"split reduce {key(dtype)} N={N}")


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_split_workload_and_layouts(dtype):
    """64 rows of 262144 (the auto split), padded pitch, rows at an odd
    offset, and the result bitwise reproducible for a given split count."""
    x = rowgen.randn(64, 262144, seed=1004, scale=3.0, dtype=dtype)
    xd = x.to(DEV)
    assert rk.rk_row_reduce_auto_splits(64, 262144, rk.RK_F32 if dtype == torch.float32
                                        else rk.RK_BF16) > 1
    err = check_split(x, xd, dtype, 0, "64x262144")
    say(f"split row_sum {key(dtype)} 64x262144 err={err:.3e}")
    a, b = rk.rk_row_sum_ex(xd), rk.rk_row_sum_ex(xd)
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(a.view(bits), b.view(bits))
    M, N, ld = 37, 30001, 30080
    xb = rowgen.randn(M, ld, seed=1005, dtype=dtype)
    for S in (0, 5, 64):
        check_split(xb[:, :N], xb.to(DEV)[:, :N], dtype, S, "pitch")
    flat = rowgen.randn(1, M * N + 3, seed=1006, dtype=dtype)[0]
    for S in (0, 5, 64):
        check_split(flat[3:].view(M, N), flat.to(DEV)[3:].view(M, N), dtype, S, "offset")


def test_split_special_rows():
    """NaN, -inf and +inf in one chunk only, an all -inf row, exact
    cancellation across chunks; and a caller's workspace reused."""
    x = rowgen.randn(6, 100000, seed=102)
    x[0, 70000] = math.nan
    x[1, :] = -math.inf
    x[2, 99999] = math.inf
    x[3, :50000] = 0.25
    x[3, 50000:] = -0.25  # each chunk's sum cancels with another's
    x[4, 10:20] = -math.inf
    xd = x.to(DEV)
    ws = torch.empty(rk.rk_row_reduce_workspace_bytes(6, 100000, 16, rk.RK_F32),
                     dtype=torch.uint8, device=DEV)
    for _ in range(2):
        m = rk.rk_row_max_ex(xd, num_splits=16, workspace=ws).cpu().numpy()
        assert np.isnan(m[0]) and m[1] == -np.inf and m[2] == np.inf
        assert m[3] == 0.25 and m[4] == x[4].max().item()
        s = rk.rk_row_sum_ex(xd, num_splits=16, workspace=ws).cpu().numpy()
        assert np.isnan(s[0]) and s[1] == -np.inf and s[2] == np.inf and s[3] == 0.0
        assert s[4] == -np.inf
        ref = oracle.row_sum(x[5:])
        assert abs(s[5] - ref[0]) <= 1e-5 * x[5].abs().sum().item()
    e = torch.empty(0, 10, device=DEV)
    assert rk.rk_row_sum_ex(e, num_splits=4).shape == (0,)


# ----------------------------------------------------------------- GeLU


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("gelu", ["tanh", "erf"])
def test_gelu_flat_and_rows(dtype, gelu):
    ref_fn = oracle.gelu_tanh if gelu == "tanh" else oracle.gelu_erf
    for M, N in ((4096, 768), (3, 1001), (1, 5), (1, 1 << 20), (257, 4095)):
        x = rowgen.randn(M, N, seed=M + N, scale=4.0, dtype=dtype)
        y = rk.rk_gelu(x.to(DEV), gelu=gelu)
        ref = ref_fn(x.double().numpy())
        assert rel_err_floor1(y, ref) <= tol_of(dtype), (M, N)
    # padded pitch (the row kernel), misaligned rows (element-wise), in place
    M, N, ld = 33, 1000, 1040
    xb = rowgen.randn(M, ld, seed=103, scale=4.0, dtype=dtype)
    canary = -12288.0
    buf = torch.full((M, 1064), canary, dtype=dtype, device=DEV)
    rk.rk_gelu(xb.to(DEV)[:, :N], gelu=gelu, out=buf[:, :N])
    assert rel_err_floor1(buf[:, :N], ref_fn(xb[:, :N].double().numpy())) <= tol_of(dtype)
    assert torch.all(buf[:, N:].cpu().float() == canary)
    flat = rowgen.randn(1, M * N + 1, seed=104, scale=4.0, dtype=dtype)[0]
    y = rk.rk_gelu(flat.to(DEV)[1:].view(M, N), gelu=gelu)
    assert rel_err_floor1(y, ref_fn(flat[1:].view(M, N).double().numpy())) <= tol_of(dtype)
    xi = xb.to(DEV)
    rk.rk_gelu(xi, gelu=gelu, out=xi)
    assert rel_err_floor1(xi, ref_fn(xb.double().numpy())) <= tol_of(dtype)


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("off", [1, 3, 5])
def test_gelu_shared_offset(dtype, off):
    """Input and output `off` elements into their buffers: the flat kernel
    (contiguous) and the row kernel (odd pitch) read and write aligned
    vectors from that offset; the bytes around the output stay untouched."""
    canary = -12288.0
    for M, N, ld in ((1, 7, 7), (5, 1001, 1001), (1, 100003, 100003), (37, 999, 1003)):
        x = rowgen.randn(M, ld, seed=off * 100 + N, scale=4.0, dtype=dtype)
        xbuf = torch.zeros(M * ld + off + 8, dtype=dtype, device=DEV)
        xbuf[off:off + M * ld] = x.reshape(-1).to(DEV)
        xd = xbuf[off:off + M * ld].view(M, ld)[:, :N]
        ybuf = torch.full((M * ld + off + 8,), canary, dtype=dtype, device=DEV)
        yd = ybuf[off:off + M * ld].view(M, ld)[:, :N]
        say(f"gelu offset {off} {key(dtype)} M={M} N={N} ld={ld}")
        rk.rk_gelu(xd, out=yd)
        assert rel_err_floor1(yd, oracle.gelu_tanh(x[:, :N].double().numpy())) <= tol_of(dtype)
        host = ybuf.cpu().float()
        assert torch.all(host[:off] == canary) and torch.all(host[off + M * ld:] == canary)
        assert torch.all(host[off:off + M * ld].view(M, ld)[:, N:] == canary)


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("off", [0, 1, 3, 7])
def test_reductions_at_offsets(dtype, off):
    """Rows at every offset (odd N, and a view `off` elements into its
    buffer): loads as aligned vectors with masked ends."""
    for M, N in ((1, 1), (9, 3), (70, 301), (33, 4097), (5, 70001)):
        flat = rowgen.randn(1, M * N + off, seed=off * 7 + N, dtype=dtype)[0]
        check_reductions(flat[off:].view(M, N), flat.to(DEV)[off:].view(M, N), dtype,
                         ("offset", off, M, N))


def test_gelu_extremes():
    z = torch.tensor([[0.0, -0.0, 1e-30, -1e-30, 10.0, 20.0, 80.0, -10.0, -30.0, -80.0, 3e38,
                       -3e38]], dtype=torch.float32)
    for gelu, fn in (("tanh", oracle.gelu_tanh), ("erf", oracle.gelu_erf)):
        y = rk.rk_gelu(z.to(DEV), gelu=gelu).cpu()
        assert torch.all(torch.isfinite(y)), (gelu, y)
        assert rel_err_floor1(y[:, :10], fn(z[:, :10].double().numpy())) <= 1e-6, gelu
        assert y[0, 10] == 3e38 and y[0, 11] == 0.0, (gelu, y)
