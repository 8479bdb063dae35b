"""Seeded random shapes and memory layouts for every row entry point, against
the CPU oracle ("Triton Kernel 实现练习" §2.2-§2.5, §4.1, §4.2, §4.3).

Each case draws a dtype, a row count, a row length (short, register-tile,
past the tiles, long rows in few rows) and a layout: contiguous, input and
output at one shared offset with padded pitches (rows at their own phases),
input and output at different offsets (element access), or in place.  The
output buffer is filled with a canary first; every element outside the
output rows must keep it.  Together the cases reach the register tiles and
their phased forms, the streaming kernels, the split kernels with a
workspace and with the partials kept in the output, and the element path.
Error measures and tolerances as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_amd as rk
import rowgen
from tolerance import TOL, rel_err, rel_err_floor1, rel_err_softmax, rel_err_sum

pytestmark = pytest.mark.gpu
EPS = float(np.float32(1e-5))
DEV = "cuda"
CANARY = -3.0
LENGTHS = [1, 7, 64, 300, 768, 1000, 3001, 4096, 12001, 16385, 33000, 65536, 100003, 262144]
ROWS = [1, 2, 3, 7, 64, 129, 300]
LAYOUTS = ["contiguous", "shared_offset", "different_offsets", "in_place"]


def _cases(n=160, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        N = int(rng.choice(LENGTHS))
        M = int(rng.choice(ROWS))
        if M * N > 2_500_000:
            continue
        dtype = "f32" if rng.random() < 0.5 else "bf16"
        layout = str(rng.choice(LAYOUTS))
        out.append((len(out), dtype, M, N, layout))
    return out


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rk.load()
    yield
    torch.cuda.synchronize()


def _strided(buf, off, M, N, ld):
    return buf[off:off + (M - 1) * ld + N].as_strided((M, N), (ld, 1))


def _layout(x, layout, seed):
    """(input view on the GPU, output view, output buffer, output offset,
    output pitch) for host rows x."""
    M, N = x.shape
    rng = np.random.default_rng(seed)
    E = 4 if x.dtype == torch.float32 else 8
    if layout == "contiguous":
        xo, yo, ldx, ldy = 0, 0, N, N
    elif layout == "shared_offset":
        o = int(rng.integers(1, E))
        pad = int(rng.integers(0, 3)) * E
        xo, yo, ldx, ldy = o, o, N + pad, N + pad + E * int(rng.integers(0, 2))
    elif layout == "different_offsets":
        xo, yo = 1, 2
        ldx, ldy = N + int(rng.integers(0, 5)), N + int(rng.integers(0, 5))
    else:
        xo, yo, ldx, ldy = 0, 0, N, N
    xbuf = torch.full((xo + (M - 1) * ldx + N + 16,), CANARY, dtype=x.dtype)
    _strided(xbuf, xo, M, N, ldx).copy_(x)
    xbuf = xbuf.to(DEV)
    xd = _strided(xbuf, xo, M, N, ldx)
    if layout == "in_place":
        return xd, xd, xbuf, xo, ldx
    ybuf = torch.full((yo + (M - 1) * ldy + N + 16,), CANARY, dtype=x.dtype, device=DEV)
    return xd, _strided(ybuf, yo, M, N, ldy), ybuf, yo, ldy


def _gaps_untouched(ybuf, off, M, N, ld):
    host = ybuf.cpu()
    mask = torch.ones(host.numel(), dtype=torch.bool)
    for r in range(M):
        mask[off + r * ld:off + r * ld + N] = False
    return bool(torch.all(host[mask].float() == CANARY))


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-{c[4]}")
def test_random_layout(case):
    idx, dt, M, N, layout = case
    dtype = torch.float32 if dt == "f32" else torch.bfloat16
    tol = TOL[dt]
    x = rowgen.randn(M, N, seed=1000 + idx, scale=3.0, dtype=dtype)
    x[::3] += 25.0  # LayerNorm rows far from zero
    res = rowgen.randn(M, N, seed=2000 + idx, dtype=dtype)
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(3000 + idx), dtype)
    wd, bd = w.to(DEV), b.to(DEV)
    print(f"case {idx}: {dt} M={M} N={N} {layout}", flush=True)

    ref = oracle.softmax(x)
    xd, yd, ybuf, yo, ldy = _layout(x, layout, idx)
    rk.rk_softmax(xd, out=yd)
    assert rel_err_softmax(yd, ref) <= tol, "softmax"
    if layout != "in_place":
        assert _gaps_untouched(ybuf, yo, M, N, ldy), "softmax gaps"

    S = [0, 2, 5][idx % 3]
    xd, yd, ybuf, yo, ldy = _layout(x, layout, idx)
    rk.rk_online_softmax(xd, num_splits=S, out=yd)
    assert rel_err_softmax(yd, ref) <= tol, ("online", S)
    if layout != "in_place":
        assert _gaps_untouched(ybuf, yo, M, N, ldy), "online gaps"

    ref = oracle.layernorm_gelu(x, w, b, EPS)
    xd, yd, ybuf, yo, ldy = _layout(x, layout, idx)
    rk.rk_layernorm_gelu(xd, wd, bd, EPS, out=yd)
    assert rel_err_floor1(yd, ref) <= tol, "layernorm"
    if layout != "in_place":
        assert _gaps_untouched(ybuf, yo, M, N, ldy), "layernorm gaps"

    ref = oracle.rmsnorm(x, w, EPS)
    xd, yd, ybuf, yo, ldy = _layout(x, layout, idx)
    rk.rk_rmsnorm(xd, wd, EPS, out=yd)
    assert rel_err(yd, ref) <= tol, "rmsnorm"
    if layout != "in_place":
        assert _gaps_untouched(ybuf, yo, M, N, ldy), "rmsnorm gaps"

    # fused residual RMSNorm, residual_out over the residual; y as above
    _, r_ref = oracle.residual_rmsnorm(x, res, w, EPS)
    y_ref = oracle.rmsnorm(torch.from_numpy(np.ascontiguousarray(r_ref)).to(dtype), w, EPS)
    xd, yd, ybuf, yo, ldy = _layout(x, layout, idx)
    rd = res.to(DEV)
    if layout == "in_place":
        rk.rk_residual_rmsnorm(xd, rd, wd, EPS, out=xd, residual_out=rd)
        yd = xd
    else:
        rk.rk_residual_rmsnorm(xd, rd, wd, EPS, out=yd, residual_out=rd)
        assert _gaps_untouched(ybuf, yo, M, N, ldy), "residual rmsnorm gaps"
    assert rel_err(rd, r_ref) <= tol, "residual_out"
    assert rel_err(yd, y_ref) <= tol, "residual rmsnorm"

    # row sum and max, one workgroup per row or split (the input at the
    # case's offset and pitch)
    S = [0, 1, 3][idx % 3]
    xd = _layout(x, layout, idx)[0]
    s_got = rk.rk_row_sum_ex(xd, num_splits=S)
    assert rel_err_sum(s_got, oracle.row_sum(x), x.double().numpy()) <= tol, ("row sum", S)
    m_got = rk.rk_row_max_ex(xd, num_splits=S).cpu().double().numpy()
    assert np.array_equal(m_got, oracle.row_max(x)), ("row max", S)
