"""Parity of rk_rmsnorm and rk_residual_rmsnorm with the CPU oracle
("Triton Kernel 实现练习" §4.2 "RMSNorm", §4.3 "Fused Residual RMSNorm").

Inputs: the workloads' x and w (rowgen) and rowgen.residual.  The fused
variant's output is the RMSNorm of residual_out as stored (the page composes
an add, then a norm of its result), so its reference is the oracle's
residual_out rounded to the storage dtype, then the oracle's RMSNorm of that.
Error measure: pure relative error, 1e-5 fp32 and 1e-2 bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_amd as rk
import rowgen
from tolerance import TOL, rel_err

pytestmark = pytest.mark.gpu
EPS = float(np.float32(1e-5))
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


def stored(a, dtype):
    """An oracle array rounded to the storage dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype)


def residual_refs(x, res, w, dtype):
    """(y, residual_out) references: residual_out from the oracle, y the
    oracle's RMSNorm of residual_out as stored."""
    _, r = oracle.residual_rmsnorm(x, res, w, EPS)
    return oracle.rmsnorm(stored(r, dtype), w, EPS), r


def check_residual(y, ro, x, res, w, dtype, what=""):
    y_ref, r_ref = residual_refs(x, res, w, dtype)
    ey, er = rel_err(y, y_ref), rel_err(ro, r_ref)
    assert er <= tol_of(dtype), (what, "residual_out", er)
    assert ey <= tol_of(dtype), (what, "y", ey)
    return ey, er


def weight(N, seed, dtype):
    w, _ = rowgen.ln_params(N, torch.Generator().manual_seed(seed), dtype)
    return w


# ----------------------------------------------------------- the workloads

WORKLOADS = ["ln_gelu_f32_4096x768", "bf16_16384x4096"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_rmsnorm_workload(name):
    d = rowgen.make(name)
    y = rk.rk_rmsnorm(d["x"].to(DEV), d["w"].to(DEV), EPS)
    err = rel_err(y, oracle.rmsnorm(d["x"], d["w"], EPS))
    say(f"rmsnorm {name} err={err:.3e}")
    assert err <= tol_of(d["x"].dtype)


@pytest.mark.parametrize("name", WORKLOADS)
def test_residual_rmsnorm_workload(name):
    d = rowgen.make(name)
    res = rowgen.residual(name)
    y, ro = rk.rk_residual_rmsnorm(d["x"].to(DEV), res.to(DEV), d["w"].to(DEV), EPS)
    ey, er = check_residual(y, ro, d["x"], res, d["w"], d["x"].dtype, name)
    say(f"residual_rmsnorm {name} err y={ey:.3e} residual_out={er:.3e}")


# ------------------------------------------------------- every tile variant


def _variant_cases(op):
    cases = []
    for dtype, code in ((torch.float32, rk.RK_F32), (torch.bfloat16, rk.RK_BF16)):
        E = 4 if code == rk.RK_F32 else 8
        for v in rk.variants(op, code):
            cap = v["max_n"]
            if v["exact"]:
                cases.append((dtype, v["index"], cap))
                continue
            for N in sorted({cap, cap - E, cap - 3 * E - 2, max(1, cap // 3 + 1)}):
                cases.append((dtype, v["index"], N))
    return cases


def _ids(v):
    return str(v).replace("torch.", "")


@pytest.mark.parametrize("dtype,index,N", _variant_cases(rk.RK_OP_RMSNORM), ids=_ids)
def test_rmsnorm_variant(dtype, index, N):
    M = 37  # the last workgroup is partial
    E = 4 if dtype == torch.float32 else 8
    ld = (N + E - 1) // E * E  # 16-byte aligned pitch; N % E != 0 exercises the tail
    base = rowgen.randn(M, ld, seed=N * 29 + index, scale=2.0, dtype=dtype)
    w = weight(N, N + index, dtype)
    y = rk.rk__rmsnorm_variant(index, base.to(DEV)[:, :N], w.to(DEV), EPS,
                               out=torch.empty(M, ld, dtype=dtype, device=DEV)[:, :N])
    assert rel_err(y, oracle.rmsnorm(base[:, :N], w, EPS)) <= tol_of(dtype)


@pytest.mark.parametrize("dtype,index,N", _variant_cases(rk.RK_OP_RESIDUAL_RMSNORM), ids=_ids)
def test_residual_rmsnorm_variant(dtype, index, N):
    M = 37
    E = 4 if dtype == torch.float32 else 8
    ld = (N + E - 1) // E * E
    base = rowgen.randn(M, ld, seed=N * 23 + index, dtype=dtype)
    rbase = rowgen.randn(M, ld, seed=N * 23 + index + 1, dtype=dtype)
    w = weight(N, N + index, dtype)
    out = torch.empty(M, ld, dtype=dtype, device=DEV)[:, :N]
    rout = torch.empty(M, ld, dtype=dtype, device=DEV)[:, :N]
    y, ro = rk.rk__residual_rmsnorm_variant(index, base.to(DEV)[:, :N], rbase.to(DEV)[:, :N],
                                            w.to(DEV), EPS, out=out, residual_out=rout)
    check_residual(y, ro, base[:, :N], rbase[:, :N], w, dtype)


def _phased_cases(op):
    """General one-row-per-group tiles on rows at every offset (odd N)."""
    cases = []
    for dtype, code in ((torch.float32, rk.RK_F32), (torch.bfloat16, rk.RK_BF16)):
        E = 4 if code == rk.RK_F32 else 8
        for v in rk.variants(op, code):
            if v["exact"] or v["rows_per_group"] != 1:
                continue
            cap = v["max_n"]
            for N in sorted({cap - E + 1, (cap // 2 + 1) | 1, 3}):
                cases.append((dtype, v["index"], N))
    return cases


@pytest.mark.parametrize("dtype,index,N", _phased_cases(rk.RK_OP_RMSNORM), ids=_ids)
def test_rmsnorm_variant_phased(dtype, index, N):
    M = 37
    x = rowgen.randn(M, N, seed=N * 11 + index, scale=2.0, dtype=dtype)
    w = weight(N, N + index + 1, dtype)
    y = rk.rk__rmsnorm_variant(index, x.to(DEV), w.to(DEV), EPS)
    assert rel_err(y, oracle.rmsnorm(x, w, EPS)) <= tol_of(dtype)


@pytest.mark.parametrize("dtype,index,N", _phased_cases(rk.RK_OP_RESIDUAL_RMSNORM), ids=_ids)
def test_residual_rmsnorm_variant_phased(dtype, index, N):
    M = 37
    x = rowgen.randn(M, N, seed=N * 7 + index, dtype=dtype)
    res = rowgen.randn(M, N, seed=N * 7 + index + 1, dtype=dtype)
    w = weight(N, N + index + 2, dtype)
    y, ro = rk.rk__residual_rmsnorm_variant(index, x.to(DEV), res.to(DEV), w.to(DEV), EPS)
    check_residual(y, ro, x, res, w, dtype, ("phased", index, N))


# ------------------------------------------------------ shapes and layouts

EDGE_N = [1, 2, 3, 63, 64, 65, 767, 769, 1000, 1025, 4095, 4097, 16384, 16385, 40000]


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_shapes(dtype, N):
    w = weight(N, N, dtype)
    wd = w.to(DEV)
    for M in (1, 257):
        say(f"rms edge {key(dtype)} M={M} N={N}")
        x = rowgen.randn(M, N, seed=M * 5 + N, scale=3.0, dtype=dtype)
        res = rowgen.randn(M, N, seed=M * 5 + N + 1, dtype=dtype)
        xd, rd = x.to(DEV), res.to(DEV)
        assert rel_err(rk.rk_rmsnorm(xd, wd, EPS), oracle.rmsnorm(x, w, EPS)) <= tol_of(dtype)
        y, ro = rk.rk_residual_rmsnorm(xd, rd, wd, EPS)
        check_residual(y, ro, x, res, w, dtype, (M, N))


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_padded_pitch_leaves_gaps_untouched(dtype):
    M, N, ldx, ldr, ldy, ldo = 33, 1000, 1040, 1008, 1064, 1024
    canary = -12288.0  # exact in fp32 and bf16
    xb = rowgen.randn(M, ldx, seed=41, scale=2.0, dtype=dtype)
    rb = rowgen.randn(M, ldr, seed=42, dtype=dtype)
    w = weight(N, 41, dtype)
    x, res, wd = xb.to(DEV)[:, :N], rb.to(DEV)[:, :N], w.to(DEV)

    def canvas(ld):
        buf = torch.full((M + 2, ld), canary, dtype=dtype, device=DEV)
        return buf, buf[1:M + 1, :N]

    def untouched(buf):
        host = buf.cpu().float()
        return (torch.all(host[0] == canary) and torch.all(host[M + 1] == canary)
                and torch.all(host[1:M + 1, N:] == canary))

    ybuf, y = canvas(ldy)
    rk.rk_rmsnorm(x, wd, EPS, out=y)
    assert rel_err(y, oracle.rmsnorm(xb[:, :N], w, EPS)) <= tol_of(dtype)
    assert untouched(ybuf)
    ybuf, y = canvas(ldy)
    obuf, ro = canvas(ldo)
    rk.rk_residual_rmsnorm(x, res, wd, EPS, out=y, residual_out=ro)
    check_residual(y, ro, xb[:, :N], rb[:, :N], w, dtype)
    assert untouched(ybuf) and untouched(obuf)


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_misaligned_and_forced_generic(dtype):
    M, N = 19, 1000
    flat = rowgen.randn(1, M * N + 1, seed=43, scale=3.0, dtype=dtype)[0]
    x = flat[1:].view(M, N)
    xd = flat.to(DEV)[1:].view(M, N)  # one element off 16-byte alignment
    res = rowgen.randn(M, N, seed=44, dtype=dtype)
    w = weight(N, 43, dtype)
    wd = w.to(DEV)
    ref = oracle.rmsnorm(x, w, EPS)
    assert rel_err(rk.rk_rmsnorm(xd, wd, EPS), ref) <= tol_of(dtype)
    y, ro = rk.rk_residual_rmsnorm(xd, res.to(DEV), wd, EPS)
    check_residual(y, ro, x, res, w, dtype, "misaligned")
    # the looping kernel on aligned data, with N beyond no tile and within one
    for n in (4099, 768):
        xa = rowgen.randn(65, n, seed=n, dtype=dtype)
        ra = rowgen.randn(65, n, seed=n + 1, dtype=dtype)
        wa = weight(n, n, dtype)
        y = rk.rk__rmsnorm_variant(-1, xa.to(DEV), wa.to(DEV), EPS)
        assert rel_err(y, oracle.rmsnorm(xa, wa, EPS)) <= tol_of(dtype)
        y, ro = rk.rk__residual_rmsnorm_variant(-1, xa.to(DEV), ra.to(DEV), wa.to(DEV), EPS)
        check_residual(y, ro, xa, ra, wa, dtype, ("generic", n))


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("N", [1, 3, 5, 301, 1001, 3001, 12001, 40001, 100001])
def test_phased_rows(dtype, N):
    """Odd N: every row at its own offset past a 16-byte boundary, shared by
    x, residual, y and residual_out row for row: the looping kernel reads
    and writes aligned vectors with masked ends and shifts the weight into
    each row's offset."""
    w = weight(N, N + 2, dtype)
    wd = w.to(DEV)
    for M in (1, 3, 70):
        x = rowgen.randn(M, N, seed=M * 5 + N, scale=2.0, dtype=dtype)
        res = rowgen.randn(M, N, seed=M * 5 + N + 1, dtype=dtype)
        say(f"rms phased {key(dtype)} M={M} N={N}")
        assert rel_err(rk.rk_rmsnorm(x.to(DEV), wd, EPS), oracle.rmsnorm(x, w, EPS)) <= tol_of(dtype)
        y, ro = rk.rk_residual_rmsnorm(x.to(DEV), res.to(DEV), wd, EPS)
        check_residual(y, ro, x, res, w, dtype, ("phased", M, N))


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_shared_offset(dtype):
    """All four matrices viewed 3 elements into their buffers (aligned pitch):
    every row at the same non-zero offset; the buffers' ends stay untouched."""
    M, N, off = 29, 2048, 3
    w = weight(N, 91, dtype)
    canary = -5.0

    def at_offset(t):
        buf = torch.full((M * N + off + 8,), canary, dtype=dtype, device=DEV)
        buf[off:off + M * N] = t.reshape(-1).to(DEV)
        return buf, buf[off:off + M * N].view(M, N)

    x = rowgen.randn(M, N, seed=92, dtype=dtype)
    res = rowgen.randn(M, N, seed=93, dtype=dtype)
    _, xd = at_offset(x)
    _, rd = at_offset(res)
    ybuf, yd = at_offset(torch.zeros(M, N, dtype=dtype))
    obuf, od = at_offset(torch.zeros(M, N, dtype=dtype))
    rk.rk_rmsnorm(xd, w.to(DEV), EPS, out=yd)
    assert rel_err(yd, oracle.rmsnorm(x, w, EPS)) <= tol_of(dtype)
    rk.rk_residual_rmsnorm(xd, rd, w.to(DEV), EPS, out=yd, residual_out=od)
    check_residual(yd, od, x, res, w, dtype, "offset")
    for buf in (ybuf, obuf):
        host = buf.cpu()
        assert torch.all(host[:off] == canary) and torch.all(host[off + M * N:] == canary)


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("N", [768, 4096, 1000, 40000, 3001])
@pytest.mark.parametrize("M", [64, 63, 1], ids=str)
def test_in_place(dtype, N, M):
    """In place, also on odd M: a two-row tile takes a missing second row as
    the first row again (read before any store, the same bytes written)."""
    x = rowgen.randn(M, N, seed=N + 7, dtype=dtype)
    res = rowgen.randn(M, N, seed=N + 8, dtype=dtype)
    w = weight(N, N, dtype)
    wd = w.to(DEV)
    xd = x.to(DEV)
    rk.rk_rmsnorm(xd, wd, EPS, out=xd)
    assert rel_err(xd, oracle.rmsnorm(x, w, EPS)) <= tol_of(dtype)
    # the residual stream updated in place, y over x
    xd, rd = x.to(DEV), res.to(DEV)
    rk.rk_residual_rmsnorm(xd, rd, wd, EPS, out=xd, residual_out=rd)
    check_residual(xd, rd, x, res, w, dtype, "y=x, residual_out=residual")
    # crossed: y over residual, residual_out over x
    xd, rd = x.to(DEV), res.to(DEV)
    rk.rk_residual_rmsnorm(xd, rd, wd, EPS, out=rd, residual_out=xd)
    check_residual(rd, xd, x, res, w, dtype, "y=residual, residual_out=x")


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("N", [768, 1000, 4096, 40000])
def test_fused_equals_add_then_norm(dtype, N):
    """y of the fused call is bitwise rk_rmsnorm of its own residual_out."""
    M = 129
    x = rowgen.randn(M, N, seed=N + 3, dtype=dtype).to(DEV)
    res = rowgen.randn(M, N, seed=N + 4, dtype=dtype).to(DEV)
    wd = weight(N, N, dtype).to(DEV)
    y, ro = rk.rk_residual_rmsnorm(x, res, wd, EPS)
    assert torch.equal(ro.cpu(), (x.cpu().float() + res.cpu().float()).to(dtype))
    y2 = rk.rk_rmsnorm(ro, wd, EPS)
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(y.view(bits), y2.view(bits))


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_special_rows(dtype):
    M, N = 6, 3000
    x = rowgen.randn(M, N, seed=47, dtype=dtype)
    x[0] = 0.0  # all zero: inv_rms = 1/sqrt(eps), y exactly 0
    x[1, :] = 0.0
    x[1, 17] = 3.0  # one nonzero: y = 3 w / sqrt(9/N + eps) there, 0 elsewhere
    x[2] *= 1e-6  # tiny row: eps dominates the mean square
    x[3] *= 1e4  # large row: eps negligible
    w = weight(N, 47, dtype)
    y = rk.rk_rmsnorm(x.to(DEV), w.to(DEV), EPS)
    yc = y.cpu().double().numpy()
    assert np.all(yc[0] == 0.0) and np.count_nonzero(yc[1]) == 1
    assert rel_err(y, oracle.rmsnorm(x, w, EPS)) <= tol_of(dtype)
    # residual cancelling x exactly: residual_out == 0, y == 0
    y, ro = rk.rk_residual_rmsnorm(x.to(DEV), (-x).to(DEV), w.to(DEV), EPS)
    assert torch.all(ro == 0) and torch.all(y == 0)


def test_deterministic_and_empty():
    d = rowgen.make("bf16_16384x4096", rows=2048)
    x, w = d["x"].to(DEV), d["w"].to(DEV)
    res = rowgen.residual("bf16_16384x4096", rows=2048).to(DEV)
    a, b = rk.rk_rmsnorm(x, w, EPS), rk.rk_rmsnorm(x, w, EPS)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    (y1, r1), (y2, r2) = (rk.rk_residual_rmsnorm(x, res, w, EPS) for _ in range(2))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16))
    e = torch.empty(0, 128, device=DEV)
    w1 = torch.ones(128, device=DEV)
    assert rk.rk_rmsnorm(e, w1, EPS).shape == (0, 128)
    y, ro = rk.rk_residual_rmsnorm(e, e.clone(), w1, EPS)
    assert y.shape == (0, 128) and ro.shape == (0, 128)


LONG_FEW = [(1, 1 << 20), (3, 100001), (6, 65536), (64, 262144)]


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("M,N", LONG_FEW)
def test_long_rows_few_rows(dtype, M, N):
    """Long rows in few rows split across workgroups, the chunk partials kept
    in y (three kernels): aligned rows and odd N; y one element into a buffer
    with 5 spare columns per row (element access), whose gaps stay untouched;
    the fused form with residual_out over the residual; in place (one kernel
    per row then).  The fused y stays bitwise the plain RMSNorm of its own
    residual_out."""
    x = rowgen.randn(M, N, seed=M + 11 * N, scale=2.0, dtype=dtype)
    res = rowgen.randn(M, N, seed=M + 11 * N + 1, dtype=dtype)
    w = weight(N, N + M, dtype)
    wd, xd, rd = w.to(DEV), x.to(DEV), res.to(DEV)
    ref = oracle.rmsnorm(x, w, EPS)
    tol = tol_of(dtype)
    say(f"rms long rows {key(dtype)} M={M} N={N}")
    assert rel_err(rk.rk_rmsnorm(xd, wd, EPS), ref) <= tol
    y, ro = rk.rk_residual_rmsnorm(xd, rd, wd, EPS)
    check_residual(y, ro, x, res, w, dtype, "split")
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(y.view(bits), rk.rk_rmsnorm(ro, wd, EPS).view(bits))
    # y at another offset than x, padded pitch
    canary = -5.0
    buf = torch.full((M, N + 5), canary, dtype=dtype, device=DEV)
    out = buf.view(-1)[1:1 + (M - 1) * (N + 5) + N].as_strided((M, N), (N + 5, 1))
    rk.rk_rmsnorm(xd, wd, EPS, out=out)
    assert rel_err(out, ref) <= tol
    flat = buf.view(-1).cpu()
    mask = torch.ones(flat.numel(), dtype=torch.bool)
    for r in range(M):
        mask[1 + r * (N + 5):1 + r * (N + 5) + N] = False
    assert torch.all(flat[mask].float() == canary)
    # residual_out over the residual, y apart
    rd2 = res.to(DEV)
    y2 = torch.empty_like(xd)
    rk.rk_residual_rmsnorm(xd, rd2, wd, EPS, out=y2, residual_out=rd2)
    check_residual(y2, rd2, x, res, w, dtype, "residual_out=residual")
    # in place: one kernel per row
    xi = x.to(DEV)
    rk.rk_rmsnorm(xi, wd, EPS, out=xi)
    assert rel_err(xi, ref) <= tol
    xi, ri = x.to(DEV), res.to(DEV)
    rk.rk_residual_rmsnorm(xi, ri, wd, EPS, out=xi, residual_out=ri)
    check_residual(xi, ri, x, res, w, dtype, "y=x")
