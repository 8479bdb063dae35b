"""Parity of rk_layernorm_gelu_ex with the CPU oracle: the exact-erf GeLU and
no activation (the LayerNorm alone) on every register tile, and rows held in
memory (the streaming kernel and the split-row pair with a Chan merge of
per-chunk (mean, M2)) with each epilogue ("Triton Kernel 实现练习" §4.1
"LayerNorm", §3.4 "Approx Activation", §6.3).

The reference is the oracle's LayerNorm + GeLU with whole-row statistics:
the split statistics compute the same function.  Error measure as for
LayerNorm + GeLU: relative error with the denominator floored at 1, 1e-5 for
fp32 and 1e-2 for bf16.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import row_wise_amd as rk
import rowgen
from tolerance import TOL, rel_err_above, rel_err_floor1

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


def ref_of(x, w, b, gelu):
    return oracle.layernorm_gelu_ex(x, w, b, EPS, gelu, 0)


def params(N, seed, dtype):
    return rowgen.ln_params(N, torch.Generator().manual_seed(seed), dtype)


# ------------------------------------------------------ exact GeLU on tiles


def _variant_cases():
    cases = []
    for dtype, code in ((torch.float32, rk.RK_F32), (torch.bfloat16, rk.RK_BF16)):
        E = 4 if code == rk.RK_F32 else 8
        for v in rk.variants(rk.RK_OP_LAYERNORM_GELU, code):
            cap = v["max_n"]
            N = cap if v["exact"] else cap - 3 * E - 2
            cases.append((dtype, v["index"], N))
    return cases


@pytest.mark.parametrize("gelu", ["erf", "none"])
@pytest.mark.parametrize("dtype,index,N", _variant_cases(),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_erf_and_plain_tile_variant(dtype, index, N, gelu):
    M = 37
    E = 4 if dtype == torch.float32 else 8
    ld = (N + E - 1) // E * E
    g = torch.Generator().manual_seed(N * 13 + index)
    base = torch.randn(M, ld, generator=g).to(dtype)
    w, b = rowgen.ln_params(N, g, dtype)
    y = rk.rk__layernorm_gelu_variant(index, base.to(DEV)[:, :N], w.to(DEV), b.to(DEV), EPS,
                                      out=torch.empty(M, ld, dtype=dtype, device=DEV)[:, :N],
                                      gelu=gelu)
    assert rel_err_floor1(y, ref_of(base[:, :N], w, b, gelu)) <= tol_of(dtype)


@pytest.mark.parametrize("name", ["ln_gelu_f32_4096x768", "bf16_16384x4096"])
def test_erf_workloads(name):
    d = rowgen.make(name)
    y = rk.rk_layernorm_gelu_ex(d["x"].to(DEV), d["w"].to(DEV), d["b"].to(DEV), EPS, gelu="erf")
    err = rel_err_floor1(y, ref_of(d["x"], d["w"], d["b"], "erf"))
    say(f"erf {name} err={err:.3e}")
    assert err <= tol_of(d["x"].dtype)
    # the tanh result differs from it by up to 4.7e-4: the kinds are not mixed up
    t = rk.rk_layernorm_gelu_ex(d["x"].to(DEV), d["w"].to(DEV), d["b"].to(DEV), EPS)
    if d["x"].dtype == torch.float32:
        assert (y - t).abs().max().item() > 1e-4


@pytest.mark.parametrize("name", ["ln_gelu_f32_4096x768", "bf16_16384x4096"])
def test_plain_layernorm_workloads(name):
    """No activation: the LayerNorm alone, also as a pure relative error
    wherever |r| >= 0.01."""
    d = rowgen.make(name)
    y = rk.rk_layernorm_gelu_ex(d["x"].to(DEV), d["w"].to(DEV), d["b"].to(DEV), EPS,
                                gelu="none")
    ref = ref_of(d["x"], d["w"], d["b"], "none")
    err = rel_err_floor1(y, ref)
    rel = rel_err_above(y, ref, 0.01)
    say(f"plain LayerNorm {name} err={err:.3e} pure relative (|r| >= 0.01) {rel:.3e}")
    assert err <= tol_of(d["x"].dtype) and rel <= tol_of(d["x"].dtype)
    # negative z is where GeLU and identity differ most: the kinds are not mixed up
    t = rk.rk_layernorm_gelu_ex(d["x"].to(DEV), d["w"].to(DEV), d["b"].to(DEV), EPS)
    assert (y - t).abs().max().item() > 0.1


# --------------------------------------------------- rows held in memory


def test_long_rows_workload():
    d = rowgen.make("ln_long_f32_64x262144")
    x, w, b = d["x"], d["w"], d["b"]
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    ref = ref_of(x, w, b, "tanh")
    for S in (1, 64, 0):
        y = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, num_splits=S)
        err = rel_err_floor1(y, ref)
        say(f"ln_long_f32_64x262144 S={S} err={err:.3e}")
        assert err <= TOL["f32"], S
    y = rk.rk_layernorm_gelu(xd, wd, bd, EPS)  # the streaming kernel
    assert rel_err_floor1(y, ref) <= TOL["f32"]
    y = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, gelu="erf", num_splits=0)
    assert rel_err_floor1(y, ref_of(x, w, b, "erf")) <= TOL["f32"]
    y = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, gelu="none", num_splits=0)
    assert rel_err_floor1(y, ref_of(x, w, b, "none")) <= TOL["f32"]


SPLIT_N = [1, 5, 1000, 4099, 16384, 16385, 40000, 100003]


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
@pytest.mark.parametrize("N", SPLIT_N)
@pytest.mark.parametrize("gelu", ["tanh", "erf", "none"])
def test_split_and_stream(dtype, N, gelu):
    w, b = params(N, N, dtype)
    wd, bd = w.to(DEV), b.to(DEV)
    for M in (1, 3, 70):
        x = rowgen.randn(M, N, seed=M * 3 + N, scale=2.0, dtype=dtype)
        x[::2] += 30.0  # mean far from zero
        xd = x.to(DEV)
        ref = ref_of(x, w, b, gelu)
        for S in (1, 2, 3, 7, 64, 0):
            say(f"ln {key(dtype)} {gelu} M={M} N={N} S={S}")
            y = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, gelu=gelu, num_splits=S)
            assert rel_err_floor1(y, ref) <= tol_of(dtype), S
        y = rk.rk__layernorm_gelu_variant(-1, xd, wd, bd, EPS, gelu=gelu)
        assert rel_err_floor1(y, ref) <= tol_of(dtype), "stream"


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_misaligned_split_and_stream(dtype):
    M, N = 9, 5001
    flat = rowgen.randn(1, M * N + 1, seed=71, scale=3.0, dtype=dtype)[0]
    x = flat[1:].view(M, N)
    xd = flat.to(DEV)[1:].view(M, N)  # one element off 16-byte alignment
    w, b = params(N, 71, dtype)
    ref = ref_of(x, w, b, "tanh")
    for S in (1, 4, 0):
        y = rk.rk_layernorm_gelu_ex(xd, w.to(DEV), b.to(DEV), EPS, num_splits=S)
        assert rel_err_floor1(y, ref) <= tol_of(dtype), S


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_split_padded_pitch_and_in_place(dtype):
    M, N, ldx, ldy = 21, 20000, 20032, 20064
    canary = -12288.0
    xb = rowgen.randn(M, ldx, seed=73, dtype=dtype)
    w, b = params(N, 73, dtype)
    x = xb.to(DEV)[:, :N]
    ref = ref_of(xb[:, :N], w, b, "tanh")
    buf = torch.full((M + 2, ldy), canary, dtype=dtype, device=DEV)
    out = buf[1:M + 1, :N]
    rk.rk_layernorm_gelu_ex(x, w.to(DEV), b.to(DEV), EPS, num_splits=5, out=out)
    assert rel_err_floor1(out, ref) <= tol_of(dtype)
    host = buf.cpu().float()
    assert torch.all(host[0] == canary) and torch.all(host[M + 1] == canary)
    assert torch.all(host[1:M + 1, N:] == canary)
    for S in (1, 6):
        xi = xb.to(DEV)[:, :N]
        rk.rk_layernorm_gelu_ex(xi, w.to(DEV), b.to(DEV), EPS, num_splits=S, out=xi)
        assert rel_err_floor1(xi, ref) <= tol_of(dtype), S


@pytest.mark.parametrize("dtype", DTYPES, ids=key)
def test_split_in_place_past_residency(dtype):
    """In place with a workspace, 96 rows x 64 chunks = 6144 workgroups, far
    more than run at once: chunk 0 of a row may be written before another
    chunk of that row starts, so the output kernel must not re-read the
    row's first element (its shift) from x.  The result equals the
    out-of-place call bit for bit and the oracle within tolerance."""
    M, N, S = 96, 65536, 64
    x = rowgen.randn(M, N, seed=83, scale=3.0, dtype=dtype)
    x[::3] += 20.0  # a shift error of O(1) is O(1) in x_hat on every row
    w, b = params(N, 83, dtype)
    wd, bd = w.to(DEV), b.to(DEV)
    ref = ref_of(x, w, b, "tanh")
    y = rk.rk_layernorm_gelu_ex(x.to(DEV), wd, bd, EPS, num_splits=S)
    xi = x.to(DEV)
    rk.rk_layernorm_gelu_ex(xi, wd, bd, EPS, num_splits=S, out=xi)
    err = rel_err_floor1(xi, ref)
    say(f"ln split in place {key(dtype)} M={M} S={S} err={err:.3e}")
    assert err <= tol_of(dtype)
    assert torch.equal(xi.cpu(), y.cpu())


def test_split_special_rows_and_determinism():
    M, N = 5, 50000
    x = rowgen.randn(M, N, seed=79)
    x[1] = 0.75  # constant row: x_hat = 0, y = GeLU(b)
    x[2, 123] = math.nan  # NaN: the whole row is NaN
    x[3, 7] = math.inf  # inf: NaN (inf - inf in the centring)
    w, b = params(N, 79, torch.float32)
    ref = ref_of(x, w, b, "tanh")
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    for S in (1, 9):
        y = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, num_splits=S).cpu().double().numpy()
        assert rel_err_floor1(y[[0, 1, 4]], ref[[0, 1, 4]]) <= TOL["f32"], S
        assert np.all(np.isnan(y[2])) and np.all(np.isnan(y[3])), S
    a = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, num_splits=9)
    c = rk.rk_layernorm_gelu_ex(xd, wd, bd, EPS, num_splits=9)
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))
