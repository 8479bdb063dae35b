"""Parity of the HIP path with the CPU oracle, element by element, on seeded
inputs.  Every call goes through the C ABI (ctypes binding in row_wise_amd).

Tolerances (tests/tolerance.py): softmax family max relative error 1e-5 for
fp32, 1e-2 for bf16 storage; LayerNorm + GeLU relative error with the
denominator floored at 1, same bounds.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import row_wise_amd as rk
import rowgen
from tolerance import TOL, rel_err, rel_err_above, rel_err_floor1, rel_err_softmax

pytestmark = pytest.mark.gpu
EPS = float(np.float32(1e-5))
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rk.load()
    yield
    torch.cuda.synchronize()


def tol_of(dtype):
    return TOL["f32"] if dtype == torch.float32 else TOL["bf16"]


def key(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


def say(msg):
    print(msg, flush=True)


# ----------------------------------------------------------- the workloads


def test_tiny_f32_64x768():
    d = rowgen.make("tiny_f32_64x768")
    x = d["x"].to(DEV)
    y = rk.rk_softmax(x)
    assert rel_err_softmax(y, oracle.softmax(d["x"])) <= TOL["f32"]
    z = rk.rk_layernorm_gelu(x, d["w"].to(DEV), d["b"].to(DEV), EPS)
    assert rel_err_floor1(z, oracle.layernorm_gelu(d["x"], d["w"], d["b"], EPS)) <= TOL["f32"]


def test_ln_gelu_f32_4096x768():
    d = rowgen.make("ln_gelu_f32_4096x768")
    y = rk.rk_layernorm_gelu(d["x"].to(DEV), d["w"].to(DEV), d["b"].to(DEV), EPS)
    ref = oracle.layernorm_gelu(d["x"], d["w"], d["b"], EPS)
    err = rel_err_floor1(y, ref)
    say(f"ln_gelu_f32_4096x768 err={err:.3e}")
    assert err <= TOL["f32"]


@pytest.mark.parametrize("name,rows", [("ln_gelu_f32_4096x768", None), ("bf16_16384x4096", 2048)])
def test_layernorm_gelu_pure_relative(name, rows):
    """The stated tolerance as a pure relative error wherever the output is
    not near zero (|r| >= 0.01), on the LayerNorm+GeLU workloads; the pure
    relative error down to |r| >= 0.001 is printed beside it."""
    d = rowgen.make(name, rows=rows)
    x, w, b = d["x"], d["w"], d["b"]
    y = rk.rk_layernorm_gelu(x.to(DEV), w.to(DEV), b.to(DEV), EPS)
    ref = oracle.layernorm_gelu(x, w, b, EPS)
    tol = tol_of(x.dtype)
    e2, e3 = rel_err_above(y, ref, 1e-2), rel_err_above(y, ref, 1e-3)
    say(f"{name} pure relative: |r| >= 1e-2 {e2:.3e}, |r| >= 1e-3 {e3:.3e}, "
        f"floor 1 {rel_err_floor1(y, ref):.3e}")
    assert e2 <= tol


def test_softmax_f32_8192x1000():
    d = rowgen.make("softmax_f32_8192x1000")
    x = d["x_softmax"]
    y = rk.rk_softmax(x.to(DEV))
    ref = oracle.softmax(x)
    err = rel_err_softmax(y, ref)
    say(f"softmax_f32_8192x1000 err={err:.3e}")
    assert err <= TOL["f32"]
    # the +1000 rows are as accurate as the others
    assert rel_err_softmax(y[::16], ref[::16]) <= TOL["f32"]


@pytest.mark.parametrize("splits", [1, 64, 0])
def test_online_f32_64x262144(splits):
    d = rowgen.make("online_f32_64x262144")
    x = d["x_softmax"]
    y = rk.rk_online_softmax(x.to(DEV), num_splits=splits)
    err = rel_err_softmax(y, oracle.softmax(x))
    say(f"online_f32_64x262144 S={splits} err={err:.3e}")
    assert err <= TOL["f32"]


def test_softmax_long_rows_few_rows():
    """8 rows of 262144: rk_softmax splits each row across workgroups with the
    chunk partials kept in the row's own output; same kernels, same split
    count and the same bits as rk_online_softmax with a workspace."""
    d = rowgen.make("online_f32_64x262144", rows=8)
    x = d["x_softmax"]
    xd = x.to(DEV)
    y = rk.rk_softmax(xd)
    assert rel_err_softmax(y, oracle.softmax(x)) <= TOL["f32"]
    S = rk.rk_online_softmax_auto_splits(8, 262144, rk.RK_F32)
    assert S > 1
    assert torch.equal(y, rk.rk_online_softmax(xd, num_splits=S))


OUT_SPLIT_CASES = [(1, 1 << 20), (3, 40001), (5, 30000), (64, 65536), (200, 12288)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
@pytest.mark.parametrize("M,N", OUT_SPLIT_CASES)
def test_partials_in_output(dtype, M, N):
    """rk_softmax and rk_layernorm_gelu on long rows in few rows keep the split
    partials inside each output row's first chunk (one bf16 row of 2^20 has
    its split count lowered until they fit) and write that chunk last:
    aligned rows, rows at their own offsets (odd N), input and output at
    different offsets (element access) with padded output pitch whose gaps
    stay untouched, and in place (one kernel per row instead)."""
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(N + M), dtype)
    wd, bd = w.to(DEV), b.to(DEV)
    x = rowgen.randn(M, N, seed=M + 3 * N, scale=3.0, dtype=dtype)
    x[::2] += 20.0
    ref_s = oracle.softmax(x)
    ref_l = oracle.layernorm_gelu(x, w, b, EPS)
    tol = tol_of(dtype)
    xd = x.to(DEV)
    say(f"partials in output {key(dtype)} M={M} N={N}")
    assert rel_err_softmax(rk.rk_softmax(xd), ref_s) <= tol
    assert rel_err_floor1(rk.rk_layernorm_gelu(xd, wd, bd, EPS), ref_l) <= tol
    # output one element into a buffer with 5 spare columns per row
    canary = -5.0
    buf = torch.full((M, N + 5), canary, dtype=dtype, device=DEV)
    out = buf.view(-1)[1:1 + (M - 1) * (N + 5) + N].as_strided((M, N), (N + 5, 1))
    for name, run, ref, err in (
            ("softmax", lambda o: rk.rk_softmax(xd, out=o), ref_s, rel_err_softmax),
            ("layernorm", lambda o: rk.rk_layernorm_gelu(xd, wd, bd, EPS, out=o), ref_l,
             rel_err_floor1)):
        buf.fill_(canary)
        run(out)
        assert err(out, ref) <= tol, name
        flat = buf.view(-1).cpu()
        mask = torch.ones(flat.numel(), dtype=torch.bool)
        for r in range(M):
            mask[1 + r * (N + 5):1 + r * (N + 5) + N] = False
        assert torch.all(flat[mask].float() == canary), name
    # in place
    xi = x.to(DEV)
    rk.rk_softmax(xi, out=xi)
    assert rel_err_softmax(xi, ref_s) <= tol
    xi = x.to(DEV)
    rk.rk_layernorm_gelu(xi, wd, bd, EPS, out=xi)
    assert rel_err_floor1(xi, ref_l) <= tol


def test_bf16_16384x4096_layernorm_gelu():
    d = rowgen.make("bf16_16384x4096")
    y = rk.rk_layernorm_gelu(d["x"].to(DEV), d["w"].to(DEV), d["b"].to(DEV), EPS)
    ref = oracle.layernorm_gelu(d["x"], d["w"], d["b"], EPS)
    err = rel_err_floor1(y, ref)
    say(f"bf16 layernorm_gelu err={err:.3e}")
    assert err <= TOL["bf16"]


def test_bf16_16384x4096_softmax():
    d = rowgen.make("bf16_16384x4096")
    xs = d["x_softmax"]
    y = rk.rk_softmax(xs.to(DEV))
    ref = oracle.softmax(xs)
    err = rel_err_softmax(y, ref)
    say(f"bf16 softmax err={err:.3e}")
    assert err <= TOL["bf16"]


# ------------------------------------------------------- every tile variant


def _variant_cases(op):
    cases = []
    for dtype, code in ((torch.float32, rk.RK_F32), (torch.bfloat16, rk.RK_BF16)):
        for v in rk.variants(op, code):
            cap = v["max_n"]
            E = 4 if code == rk.RK_F32 else 8
            if v["exact"]:
                cases.append((dtype, v["index"], cap))
                continue
            for N in sorted({cap, cap - E, cap - 3 * E - 2, max(1, cap // 3 + 1)}):
                cases.append((dtype, v["index"], N))
    return cases


@pytest.mark.parametrize("dtype,index,N", _variant_cases(rk.RK_OP_SOFTMAX),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_softmax_variant(dtype, index, N):
    M = 37  # not a multiple of the rows per workgroup: the last one is partial
    E = 4 if dtype == torch.float32 else 8
    ld = (N + E - 1) // E * E  # 16-byte aligned pitch (N % E != 0 exercises the tail)
    base = rowgen.randn(M, ld, seed=N * 31 + index, scale=4.0, dtype=dtype)
    x = base.to(DEV)[:, :N]
    y = rk.rk__softmax_variant(index, x, out=torch.empty(M, ld, dtype=dtype, device=DEV)[:, :N])
    assert rel_err_softmax(y, oracle.softmax(base[:, :N])) <= tol_of(dtype)


@pytest.mark.parametrize("dtype,index,N", _variant_cases(rk.RK_OP_LAYERNORM_GELU),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_layernorm_gelu_variant(dtype, index, N):
    M = 37
    E = 4 if dtype == torch.float32 else 8
    ld = (N + E - 1) // E * E
    g = torch.Generator().manual_seed(N * 17 + index)
    base = torch.randn(M, ld, generator=g).to(dtype)
    w, b = rowgen.ln_params(N, g, dtype)
    x = base.to(DEV)[:, :N]
    y = rk.rk__layernorm_gelu_variant(index, x, w.to(DEV), b.to(DEV), EPS,
                                      out=torch.empty(M, ld, dtype=dtype, device=DEV)[:, :N])
    assert rel_err_floor1(y, oracle.layernorm_gelu(base[:, :N], w, b, EPS)) <= tol_of(dtype)


def _exact_bf16_layernorm():
    return [(v["index"], v["max_n"]) for v in rk.variants(rk.RK_OP_LAYERNORM_GELU, rk.RK_BF16)
            if v["exact"]]


@pytest.mark.parametrize("index,N", _exact_bf16_layernorm(), ids=str)
def test_layernorm_gelu_bf16_exact_hard_rows(index, N):
    """The exact bf16 tiles, one pass over x - x[0] or two passes: rows whose
    first element is far from the mean (the shift then cancels most in
    sum d^2 / N - mean_d^2), rows far from zero, a constant row, a row of two
    values and one huge outlier; within 1e-2 of the oracle."""
    g = torch.Generator().manual_seed(N + 7 * index)
    x = torch.randn(9, N, generator=g)
    x[0, 0] = 40.0  # the shift 40 sigma from the mean
    x[1, 0] = -300.0
    x[2] += 100.0  # mean 100, sigma 1 (bf16 spacing 0.5 there)
    x[3] = 1.25  # constant: x_hat = 0, y = GeLU(b)
    x[4] = torch.where(torch.arange(N) % 2 == 0, 3.0, -1.0)
    x[5] = 0.0
    x[5, N // 2] = 1000.0  # one outlier: x_hat = +-sqrt(N - 1) and -1 / sqrt(N - 1)
    x[6] *= 1e-3  # variance near eps
    x[7] = x[7] * 50.0 + 2000.0
    x = x.to(torch.bfloat16)
    w, b = rowgen.ln_params(N, g, torch.bfloat16)
    y = rk.rk__layernorm_gelu_variant(index, x.to(DEV), w.to(DEV), b.to(DEV), EPS)
    ref = oracle.layernorm_gelu(x, w, b, EPS)
    err = rel_err_floor1(y, ref)
    say(f"ln bf16 exact index {index} N={N} hard rows err={err:.2e}")
    assert err <= TOL["bf16"]


def _general_bf16_layernorm():
    """Ragged widths for every general bf16 tile: two multiples of 8 (rows on
    16-byte boundaries: the tile itself, one shifted pass or two) and, for a
    one-row tile, an odd width (rows at every offset: its phased form)."""
    cases = []
    for v in rk.variants(rk.RK_OP_LAYERNORM_GELU, rk.RK_BF16):
        if v["exact"] or v["max_n"] > 32768:
            continue
        widths = {v["max_n"] - 40, v["max_n"] // 2 + 8}
        if v["rows_per_group"] == 1:
            widths.add(v["max_n"] - 37)
        for N in sorted(widths):
            cases.append((v["index"], N))
    return cases


@pytest.mark.parametrize("index,N", _general_bf16_layernorm(), ids=str)
def test_layernorm_gelu_bf16_general_hard_rows(index, N):
    """The general bf16 tiles (one shifted pass or two passes, padded slots
    excluded) on ragged widths with the adversarial rows of the exact test,
    on 9 rows (a two-row tile's last row repeated); within 1e-2 of the
    oracle."""
    g = torch.Generator().manual_seed(N + 11 * index)
    x = torch.randn(9, N, generator=g)
    x[0, 0] = 40.0
    x[1, 0] = -300.0
    x[2] += 100.0
    x[3] = 1.25
    x[4] = torch.where(torch.arange(N) % 2 == 0, 3.0, -1.0)
    x[5] = 0.0
    x[5, N // 2] = 1000.0
    x[6] *= 1e-3
    x[7] = x[7] * 50.0 + 2000.0
    x = x.to(torch.bfloat16)
    w, b = rowgen.ln_params(N, g, torch.bfloat16)
    y = rk.rk__layernorm_gelu_variant(index, x.to(DEV), w.to(DEV), b.to(DEV), EPS)
    ref = oracle.layernorm_gelu(x, w, b, EPS)
    err = rel_err_floor1(y, ref)
    say(f"ln bf16 general index {index} N={N} hard rows err={err:.2e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("index,N", _exact_bf16_layernorm(), ids=str)
def test_layernorm_gelu_bf16_exact_many_rows(index, N):
    """Every exact bf16 tile on an odd number of rows (up to 5001, 2^26
    elements at most): the persistent forms then loop several times per
    workgroup, through both halves of their unrolled loop and with the
    prefetch past the last row.  Sampled rows (the first and last 64 and 128
    seeded others) within 1e-2 of the oracle; the rest finite."""
    M = min(5001, (1 << 26) // N) | 1
    g = torch.Generator().manual_seed(3 * N + index)
    x = (torch.randn(M, N, generator=g) * 1.5 + 0.25).to(torch.bfloat16)
    w, b = rowgen.ln_params(N, g, torch.bfloat16)
    xd = x.to(DEV)
    y = rk.rk__layernorm_gelu_variant(index, xd, w.to(DEV), b.to(DEV), EPS)
    assert bool(torch.isfinite(y.float()).all())
    rows = torch.cat([torch.arange(64), torch.arange(M - 64, M),
                      torch.randint(64, M - 64, (128,), generator=g)]).unique()
    ref = oracle.layernorm_gelu(x[rows], w, b, EPS)
    err = rel_err_floor1(y[rows.to(DEV)], ref)
    say(f"ln bf16 exact index {index} N={N} M={M} sampled err={err:.2e}")
    assert err <= TOL["bf16"]


def _phased_cases(op):
    """General one-row-per-group tiles on rows at every offset: odd N, so row
    r starts r N elements into an aligned buffer; N + E - 1 fits the tile."""
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


@pytest.mark.parametrize("dtype,index,N", _phased_cases(rk.RK_OP_SOFTMAX),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_softmax_variant_phased(dtype, index, N):
    M = 37
    x = rowgen.randn(M, N, seed=N * 13 + index, scale=4.0, dtype=dtype)
    y = rk.rk__softmax_variant(index, x.to(DEV))
    assert rel_err_softmax(y, oracle.softmax(x)) <= tol_of(dtype)


@pytest.mark.parametrize("dtype,index,N", _phased_cases(rk.RK_OP_LAYERNORM_GELU),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_layernorm_gelu_variant_phased(dtype, index, N):
    M = 37
    g = torch.Generator().manual_seed(N * 19 + index)
    x = (torch.randn(M, N, generator=g) + 5.0).to(dtype)
    w, b = rowgen.ln_params(N, g, dtype)
    for gelu in ("tanh", "erf", "none"):
        y = rk.rk__layernorm_gelu_variant(index, x.to(DEV), w.to(DEV), b.to(DEV), EPS, gelu=gelu)
        ref = (oracle.layernorm_gelu(x, w, b, EPS) if gelu == "tanh"
               else oracle.layernorm_gelu_ex(x, w, b, EPS, gelu))
        assert rel_err_floor1(y, ref) <= tol_of(dtype), gelu


# ------------------------------------------------------ shapes and layouts

EDGE_N = [1, 2, 3, 63, 64, 65, 767, 769, 1000, 1025, 4095, 4097, 16384, 16385, 40000]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_shapes(dtype, N):
    tol = tol_of(dtype)
    for M in (1, 257):
        say(f"edge {key(dtype)} M={M} N={N}")
        x = rowgen.randn(M, N, seed=M * 7 + N, scale=3.0, dtype=dtype)
        xd = x.to(DEV)
        ref = oracle.softmax(x)
        assert rel_err_softmax(rk.rk_softmax(xd), ref) <= tol
        for S in (1, 3, 0):
            assert rel_err_softmax(rk.rk_online_softmax(xd, num_splits=S), ref) <= tol, S
        g = torch.Generator().manual_seed(N)
        w, b = rowgen.ln_params(N, g, dtype)
        y = rk.rk_layernorm_gelu(xd, w.to(DEV), b.to(DEV), EPS)
        assert rel_err_floor1(y, oracle.layernorm_gelu(x, w, b, EPS)) <= tol


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
def test_padded_pitch_leaves_gaps_untouched(dtype):
    M, N, ldx, ldy = 33, 1000, 1040, 1064
    canary = -12288.0  # exact in fp32 and bf16
    xb = rowgen.randn(M, ldx, seed=5, scale=2.0, dtype=dtype)
    x = xb.to(DEV)[:, :N]
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(5), dtype)
    checks = [
        ("softmax", lambda o: rk.rk_softmax(x, out=o), oracle.softmax(xb[:, :N]),
         rel_err_softmax),
        ("online S=4", lambda o: rk.rk_online_softmax(x, num_splits=4, out=o),
         oracle.softmax(xb[:, :N]), rel_err_softmax),
        ("layernorm_gelu", lambda o: rk.rk_layernorm_gelu(x, w.to(DEV), b.to(DEV), EPS, out=o),
         oracle.layernorm_gelu(xb[:, :N], w, b, EPS), rel_err_floor1),
    ]
    for name, fn, ref, measure in checks:
        buf = torch.full((M + 2, ldy), canary, dtype=dtype, device=DEV)
        out = buf[1:M + 1, :N]
        fn(out)
        assert measure(out, ref) <= tol_of(dtype), name
        host = buf.cpu().float()
        assert torch.all(host[0] == canary) and torch.all(host[M + 1] == canary), name
        assert torch.all(host[1:M + 1, N:] == canary), name


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
def test_misaligned_base_takes_elementwise_path(dtype):
    M, N = 19, 1000
    flat = rowgen.randn(1, M * N + 1, seed=9, scale=3.0, dtype=dtype)[0]
    xd = flat.to(DEV)[1:].view(M, N)  # one element off 16-byte alignment
    x = flat[1:].view(M, N)
    ref = oracle.softmax(x)
    assert rel_err_softmax(rk.rk_softmax(xd), ref) <= tol_of(dtype)
    assert rel_err_softmax(rk.rk_online_softmax(xd, num_splits=5), ref) <= tol_of(dtype)
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(9), dtype)
    y = rk.rk_layernorm_gelu(xd, w.to(DEV), b.to(DEV), EPS)
    assert rel_err_floor1(y, oracle.layernorm_gelu(x, w, b, EPS)) <= tol_of(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
def test_generic_paths_forced(dtype):
    M, N = 65, 4099
    x = rowgen.randn(M, N, seed=11, scale=3.0, dtype=dtype)
    xd = x.to(DEV)
    assert rel_err_softmax(rk.rk__softmax_variant(-1, xd), oracle.softmax(x)) <= tol_of(dtype)
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(11), dtype)
    y = rk.rk__layernorm_gelu_variant(-1, xd, w.to(DEV), b.to(DEV), EPS)
    assert rel_err_floor1(y, oracle.layernorm_gelu(x, w, b, EPS)) <= tol_of(dtype)


STREAM_N = [1, 5, 300, 1000, 3000, 9000, 40000, 100003]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
@pytest.mark.parametrize("N", STREAM_N)
def test_stream_widths(dtype, N):
    """The one-workgroup-per-row kernels take 1, 4 or 16 waves per row by N,
    and pack one-wave rows four to a workgroup: row counts that are not a
    multiple of four, on the vector (aligned) and element (misaligned) paths."""
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(N), dtype)
    wd, bd = w.to(DEV), b.to(DEV)
    for M in (1, 3, 70):
        flat = rowgen.randn(1, M * N + 1, seed=M + N, scale=3.0, dtype=dtype)[0]
        x = flat[1:].view(M, N)
        ref_s = oracle.softmax(x)
        ref_l = oracle.layernorm_gelu(x, w, b, EPS)
        aligned = x.contiguous().to(DEV)
        misaligned = flat.to(DEV)[1:].view(M, N)  # one element off 16-byte alignment
        for name, xd in (("aligned", aligned), ("misaligned", misaligned)):
            say(f"stream {key(dtype)} M={M} N={N} {name}")
            y = rk.rk__softmax_variant(-1, xd) if name == "aligned" else rk.rk_softmax(xd)
            assert rel_err_softmax(y, ref_s) <= tol_of(dtype), name
            y = (rk.rk__layernorm_gelu_variant(-1, xd, wd, bd, EPS) if name == "aligned"
                 else rk.rk_layernorm_gelu(xd, wd, bd, EPS))
            assert rel_err_floor1(y, ref_l) <= tol_of(dtype), name


PHASE_N = [1, 3, 5, 301, 1001, 3001, 12001, 40001, 100001]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
@pytest.mark.parametrize("N", PHASE_N)
def test_phased_rows(dtype, N):
    """Odd N: row r starts r N elements into an aligned buffer, so each row
    sits at its own offset past a 16-byte boundary; input and output share it
    row for row, and the rows-in-memory kernels read and write them as aligned
    vectors with masked ends (streaming and split)."""
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(N + 1), dtype)
    wd, bd = w.to(DEV), b.to(DEV)
    for M in (1, 3, 70):
        x = rowgen.randn(M, N, seed=M * 7 + N, scale=3.0, dtype=dtype)
        x[::2] += 30.0  # LayerNorm rows far from zero
        xd = x.to(DEV)
        ref_s = oracle.softmax(x)
        ref_l = oracle.layernorm_gelu(x, w, b, EPS)
        say(f"phased {key(dtype)} M={M} N={N}")
        assert rel_err_softmax(rk.rk_softmax(xd), ref_s) <= tol_of(dtype)
        assert rel_err_floor1(rk.rk_layernorm_gelu(xd, wd, bd, EPS), ref_l) <= tol_of(dtype)
        # 64 splits of short rows leave most chunks empty, and the last one
        # takes the row's end past the chunk grid
        for S in (2, 3, 7, 64, 0):
            y = rk.rk_online_softmax(xd, num_splits=S)
            assert rel_err_softmax(y, ref_s) <= tol_of(dtype), S
            y = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, num_splits=S)
            assert rel_err_floor1(y, ref_l) <= tol_of(dtype), S


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
@pytest.mark.parametrize("off", [1, 3])
def test_shared_offset_and_in_place(dtype, off):
    """Every row at the same non-zero offset (input and output views `off`
    elements into their buffers, aligned pitch), then in place over odd N."""
    M, N = 37, 4096
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(off), dtype)
    wd, bd = w.to(DEV), b.to(DEV)
    flat = rowgen.randn(1, M * N + off, seed=off + 50, scale=2.0, dtype=dtype)[0]
    x = flat[off:].view(M, N)
    xd = flat.to(DEV)[off:].view(M, N)
    canary = -7.0
    obuf = torch.full((M * N + off + 8,), canary, dtype=dtype, device=DEV)
    out = obuf[off:off + M * N].view(M, N)
    rk.rk_softmax(xd, out=out)
    assert rel_err_softmax(out, oracle.softmax(x)) <= tol_of(dtype)
    rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, num_splits=4, out=out)
    assert rel_err_floor1(out, oracle.layernorm_gelu(x, w, b, EPS)) <= tol_of(dtype)
    host = obuf.cpu()
    assert torch.all(host[:off] == canary) and torch.all(host[off + M * N:] == canary)
    # in place, odd N
    M, N = 33, 2999
    x = rowgen.randn(M, N, seed=off + 60, scale=2.0, dtype=dtype)
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(off + 1), dtype)
    xd = x.to(DEV)
    rk.rk_softmax(xd, out=xd)
    assert rel_err_softmax(xd, oracle.softmax(x)) <= tol_of(dtype)
    xd = x.to(DEV)
    rk.rk_layernorm_gelu(xd, w.to(DEV), b.to(DEV), EPS, out=xd)
    assert rel_err_floor1(xd, oracle.layernorm_gelu(x, w, b, EPS)) <= tol_of(dtype)
    xd = x.to(DEV)
    rk.rk_online_softmax(xd, num_splits=5, out=xd)
    assert rel_err_softmax(xd, oracle.softmax(x)) <= tol_of(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
def test_phased_rows_different_pitches(dtype):
    """Input pitch N + 6 and output pitch N + 6 + E: the two differ by one
    16-byte vector, so every row's offset is the same in both though the
    pitches are odd and unequal; the gaps between output rows stay untouched."""
    E = 4 if dtype == torch.float32 else 8
    M, N = 41, 1003
    ldx, ldy = N + 6, N + 6 + E
    canary = -9.0
    xb = rowgen.randn(M, ldx, seed=E + 70, scale=3.0, dtype=dtype)
    x = xb[:, :N]
    w, b = rowgen.ln_params(N, torch.Generator().manual_seed(E + 71), dtype)
    xd = xb.to(DEV)[:, :N]
    res = rowgen.randn(M, N, seed=E + 72, dtype=dtype)
    for name, run, ref, err in (
            ("softmax", lambda o: rk.rk_softmax(xd, out=o), oracle.softmax(x), rel_err_softmax),
            ("online", lambda o: rk.rk_online_softmax(xd, num_splits=3, out=o), oracle.softmax(x),
             rel_err_softmax),
            ("layernorm", lambda o: rk.rk_layernorm_gelu(xd, w.to(DEV), b.to(DEV), EPS, out=o),
             oracle.layernorm_gelu(x, w, b, EPS), rel_err_floor1),
            ("layernorm split", lambda o: rk.rk_layernorm_gelu_ex(xd, w.to(DEV), b.to(DEV), EPS,
                                                                   num_splits=4, out=o),
             oracle.layernorm_gelu(x, w, b, EPS), rel_err_floor1),
            ("rmsnorm", lambda o: rk.rk_rmsnorm(xd, w.to(DEV), EPS, out=o),
             oracle.rmsnorm(x, w, EPS), rel_err),
            ("gelu", lambda o: rk.rk_gelu(xd, out=o), oracle.gelu_tanh(x.double().numpy()),
             rel_err_floor1)):
        buf = torch.full((M, ldy), canary, dtype=dtype, device=DEV)
        run(buf[:, :N])
        assert err(buf[:, :N], ref) <= tol_of(dtype), name
        assert torch.all(buf[:, N:].cpu().float() == canary), name


def test_in_place():
    M, N = 64, 768
    d = rowgen.make("tiny_f32_64x768")
    x = d["x"].to(DEV).clone()
    rk.rk_softmax(x, out=x)
    assert rel_err_softmax(x, oracle.softmax(d["x"])) <= TOL["f32"]
    x = d["x"].to(DEV).clone()
    rk.rk_layernorm_gelu(x, d["w"].to(DEV), d["b"].to(DEV), EPS, out=x)
    assert rel_err_floor1(x, oracle.layernorm_gelu(d["x"], d["w"], d["b"], EPS)) <= TOL["f32"]
    x = rowgen.randn(8, 50000, seed=3).to(DEV)
    ref = oracle.softmax(x.cpu())
    rk.rk_online_softmax(x, num_splits=1, out=x)
    assert rel_err_softmax(x, ref) <= TOL["f32"]


@pytest.mark.parametrize("M", [1, 3, 257, 4097], ids=str)
def test_layernorm_gelu_bf16_exact_in_place_odd_rows(M):
    """The dispatched exact bf16 tiles in place on an odd number of rows: the
    two-row tile takes a missing second row as the first row again (read
    before any store, written twice with the same bytes), the persistent
    tiles prefetch past the last row.  Every row within 1e-2 of the oracle
    and equal, bit for bit, to the out-of-place call."""
    for N in (3072, 4096, 5120, 6144, 8192, 16384):
        g = torch.Generator().manual_seed(M * 31 + N)
        x = (torch.randn(M, N, generator=g) + 0.5).to(torch.bfloat16)
        w, b = rowgen.ln_params(N, g, torch.bfloat16)
        wd, bd = w.to(DEV), b.to(DEV)
        out = rk.rk_layernorm_gelu(x.to(DEV), wd, bd, EPS)
        xi = x.to(DEV)
        rk.rk_layernorm_gelu(xi, wd, bd, EPS, out=xi)
        assert torch.equal(xi.view(torch.int16), out.view(torch.int16)), N
        rows = torch.arange(M) if M <= 257 else torch.cat([torch.arange(64), torch.arange(M - 64, M)])
        err = rel_err_floor1(xi[rows.to(DEV)], oracle.layernorm_gelu(x[rows], w, b, EPS))
        say(f"ln bf16 in place M={M} N={N} err={err:.2e}")
        assert err <= TOL["bf16"]


@pytest.mark.parametrize("M", [1, 3, 257, 4097], ids=str)
def test_layernorm_gelu_f32_exact_in_place_odd_rows(M):
    """The dispatched exact fp32 tiles of two rows per group (two passes) in
    place on an odd number of rows: a missing second row is the first row
    again.  Every row within 1e-5 of the oracle and equal, bit for bit, to the
    out-of-place call."""
    for N in (1536, 2560, 3072, 4096, 5120, 6144, 8192):
        g = torch.Generator().manual_seed(M * 37 + N)
        x = torch.randn(M, N, generator=g) + 0.5
        w, b = rowgen.ln_params(N, g, torch.float32)
        wd, bd = w.to(DEV), b.to(DEV)
        out = rk.rk_layernorm_gelu(x.to(DEV), wd, bd, EPS)
        xi = x.to(DEV)
        rk.rk_layernorm_gelu(xi, wd, bd, EPS, out=xi)
        assert torch.equal(xi.view(torch.int32), out.view(torch.int32)), N
        rows = torch.arange(M) if M <= 257 else torch.cat([torch.arange(64), torch.arange(M - 64, M)])
        err = rel_err_floor1(xi[rows.to(DEV)], oracle.layernorm_gelu(x[rows], w, b, EPS))
        say(f"ln f32 in place M={M} N={N} err={err:.2e}")
        assert err <= TOL["f32"]


def _exact_f32_layernorm():
    return [(v["index"], v["max_n"]) for v in rk.variants(rk.RK_OP_LAYERNORM_GELU, rk.RK_F32)
            if v["exact"]]


@pytest.mark.parametrize("index,N", _exact_f32_layernorm(), ids=str)
def test_layernorm_gelu_f32_exact_many_rows(index, N):
    """Every exact fp32 tile on an odd number of rows (up to 4001, 2^25
    elements at most), sampled rows within 1e-5 of the oracle."""
    M = min(4001, (1 << 25) // N) | 1
    g = torch.Generator().manual_seed(5 * N + index)
    x = torch.randn(M, N, generator=g) * 1.5 + 0.25
    w, b = rowgen.ln_params(N, g, torch.float32)
    y = rk.rk__layernorm_gelu_variant(index, x.to(DEV), w.to(DEV), b.to(DEV), EPS)
    rows = torch.cat([torch.arange(64), torch.arange(M - 64, M),
                      torch.randint(64, M - 64, (128,), generator=g)]).unique()
    err = rel_err_floor1(y[rows.to(DEV)], oracle.layernorm_gelu(x[rows], w, b, EPS))
    say(f"ln f32 exact index {index} N={N} M={M} sampled err={err:.2e}")
    assert err <= TOL["f32"]


def test_deterministic():
    d = rowgen.make("bf16_16384x4096", rows=2048)
    x, w, b = (d[k].to(DEV) for k in ("x", "w", "b"))
    for fn in (lambda: rk.rk_softmax(x), lambda: rk.rk_layernorm_gelu(x, w, b, EPS),
               lambda: rk.rk_online_softmax(x, num_splits=8)):
        a, c = fn(), fn()
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
def test_infinities(dtype):
    M, N = 7, 3000
    x = rowgen.randn(M, N, seed=13, dtype=dtype)
    x[0, ::7] = -math.inf  # some -inf: those outputs are exactly 0
    x[1, :] = -math.inf  # all -inf: NaN (the definition's IEEE value)
    x[2, 5] = math.inf  # +inf: NaN
    x[3, 2999] = math.nan  # NaN anywhere: NaN
    ref = oracle.softmax(x)
    for y in (rk.rk_softmax(x.to(DEV)), rk.rk_online_softmax(x.to(DEV), num_splits=1),
              rk.rk_online_softmax(x.to(DEV), num_splits=4),
              rk.rk__softmax_variant(-1, x.to(DEV))):
        yc = y.cpu().double().numpy()
        assert np.all(yc[0, ::7] == 0.0)
        assert rel_err_softmax(yc[[0, 4, 5, 6]], ref[[0, 4, 5, 6]]) <= tol_of(dtype)
        for r in (1, 2, 3):
            assert np.all(np.isnan(yc[r])) and np.all(np.isnan(ref[r])), r


def _neg_inf_rows(dtype, N=262144):
    """Rows of 3 N(0,1) with -inf over whole blocks or chunks: the identity
    state (-inf, 0) of the online recurrence and of the chunk merge.  The
    regions are whole chunks of S = 2, 4 and 64 (N is a multiple of 64
    vectors of either format), the first 64 KiB (one streaming step of a
    16-wave workgroup), all but the last element, and every 7th element."""
    regions = [(0, 65536 // torch.tensor([], dtype=dtype).element_size()), (0, N - 1),
               (0, N // 2), (N // 2, N), (N // 4, N // 2), (3 * N // 4, N),
               (0, N // 64), (32 * N // 64, 33 * N // 64), (63 * N // 64, N)]
    x = rowgen.randn(len(regions) + 2, N, seed=97, scale=3.0, dtype=dtype)
    for i, (a, b) in enumerate(regions):
        x[i, a:b] = -math.inf
    x[len(regions), ::7] = -math.inf
    return x  # the last row stays finite


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=key)
def test_neg_inf_blocks_and_chunks(dtype):
    """Every online form against the plain definition on rows whose leading
    blocks or one chunk hold only -inf ("第 6 讲" §7.2 start state;
    "Triton Kernel 实现练习" §2.5 split version): streaming (S = 1), the
    workspace split at S = 2, 4, 64, and rk_softmax's split with the
    partials kept in the output.  -inf inputs give exact zeros."""
    x = _neg_inf_rows(dtype)
    M, N = x.shape
    ref = oracle.softmax(x)
    zero = torch.isinf(x).numpy()
    xd = x.to(DEV)
    outs = {f"S={S}": rk.rk_online_softmax(xd, num_splits=S) for S in (1, 2, 4, 64)}
    assert rk.rk_online_softmax_auto_splits(M, N, rk.RK_F32 if dtype == torch.float32
                                            else rk.RK_BF16) > 1
    outs["rk_softmax"] = rk.rk_softmax(xd)
    for name, y in outs.items():
        yc = y.cpu().double().numpy()
        err = rel_err_softmax(yc, ref)
        say(f"neg_inf {key(dtype)} {name} err={err:.3e}")
        assert np.all(yc[zero] == 0.0), name
        assert err <= tol_of(dtype), name
        assert yc[1, N - 1] == 1.0, name  # one finite value: exactly 1


def test_empty_rows_is_noop():
    x = torch.empty(0, 128, device=DEV)
    assert rk.rk_softmax(x).shape == (0, 128)
    assert rk.rk_online_softmax(x, num_splits=4).shape == (0, 128)
    w = torch.ones(128, device=DEV)
    assert rk.rk_layernorm_gelu(x, w, w, EPS).shape == (0, 128)


def test_probe_copy():
    src = torch.randn(1 << 20, device=DEV)
    dst = torch.empty_like(src)
    rk.rk_probe_copy(src, dst)
    assert torch.equal(src, dst)
    dst.zero_()
    rk.rk_probe_copy(src, dst, max_workgroups=64)
    assert torch.equal(src, dst)
