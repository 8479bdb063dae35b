"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each ``check_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` on a
violation.  ``tests/test_oracle_pins.py`` runs them against the real oracle;
``tests/test_oracle_mutants.py`` runs them against copies of the oracle with a
planted mistake and requires that some check fails for every mutant.

What pins what (citations are to the pages' titles and sections):

* softmax, "Triton Kernel 实现练习" §2.4: rows sum to 1; invariance under adding
  a constant (bitwise, for shifts exact in double); constant row -> 1/N;
  N = 2 -> logistic closed form; N = 1 -> 1; the textbook definition
  exp(x_j) / sum_k exp(x_k) evaluated by brute force at 50 digits (mpmath);
  torch.softmax in float64.
* online / split softmax, same page §2.5 and "第 6 讲" §7.2: the streaming
  recurrence reaches (max, sum exp(x - max)) for every block size; geometric
  rows whose statistics are closed-form sums; the merge has (-inf, 0) as its
  identity, is commutative and associative, and merging two halves gives the
  whole; split statistics equal the whole-row statistics for any chunk count,
  including empty chunks; a block or chunk holding only -inf has the state
  (-inf, 0) and leaves the row's statistics those of its finite values.
* LayerNorm, "Triton Kernel 实现练习" §4.1: mean(x_hat) = 0 and
  var(x_hat) = s2 / (s2 + eps); reduction to torch.nn.functional.layer_norm in
  float64; a constant row gives x_hat = 0 and y = GeLU(b); an eps-sensitive
  row pins where eps enters.
* tanh GeLU, same page §3.4: GeLU(0) = 0; GeLU(z) - GeLU(-z) = z; limits
  z and 0 at +-large z; torch.nn.functional.gelu(approximate="tanh") in
  float64; distance to the erf form peaks near 4.73e-4.
* RMSNorm, same page §4.2: torch.nn.functional.rms_norm in float64;
  mean((y / w)^2) = ms / (ms + eps); odd symmetry; a constant row in closed
  form; an eps-sensitive row against numpy's mean of squares.
* fused residual RMSNorm, same page §4.3: residual_out is x + residual
  exactly; out is RMSNorm of residual_out (torch, float64).
* exact GeLU, same page §3.4: GeLU(0) = 0; GeLU(z) - GeLU(-z) = z; z times the
  standard normal CDF at 50 digits (mpmath); torch gelu(approximate="none")
  in float64; its largest distance to the tanh form is 4.73e-4 near -2.70.
* split LayerNorm statistics (same page §6.3, reduction by parts, merged by
  Chan, Golub and LeVeque's pairwise update): arithmetic progressions in
  closed form; the merge has n = 0 as identity, is commutative and
  associative, and merging pieces gives the whole-row two-pass moments; the
  split statistics of any chunk count equal the whole row's; LayerNorm + GeLU
  on them equals the whole-row version, and with erf equals torch's
  layer_norm followed by the exact gelu.
* row sum and row max, same page §2.2 and §2.3: the sum against math.fsum
  (correctly rounded) and closed forms (arithmetic progressions, exact
  cancellation); the max against numpy, invariant under permutation, NaN
  propagating, -inf for an all -inf row.
* attention, same page §5.1-5.2 and "第 6 讲" §7: torch's
  scaled_dot_product_attention in float64 (causal and not); closed forms
  (equal value rows give that row; q = 0 averages the visible value rows;
  T = 1 returns v; the first causal row returns v[0]; a dominant score picks
  its value row); invariance of non-causal attention under a joint
  permutation of keys and values; the definition at 50 digits on tiny
  shapes; the tiled online form equals the definition for every block size.
"""
from __future__ import annotations

import math

import numpy as np

EPS = float(np.float32(1e-5))


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300)))


# ---------------------------------------------------------------- softmax


def check_softmax_sums_to_one(orc):
    for n, scale in [(7, 1.0), (768, 1.0), (1000, 4.0), (4096, 8.0), (262144, 3.0)]:
        x = scale * _rng(n).standard_normal((2, n))
        y = orc.softmax(x)
        assert np.all(y > 0), n
        err = np.abs(y.sum(axis=1) - 1.0).max()
        assert err <= 1e-13, (n, err)


def check_softmax_shift_invariance(orc):
    # values on a 2^-20 grid, |x| < 2^5: x + c and max + c are exact in double
    # for |c| <= 2^30, so x - max is formed from the same real numbers
    x = np.round(4.0 * _rng(3).standard_normal((4, 1000)) * 2.0**20) / 2.0**20
    y = orc.softmax(x)
    for c in (1000.0, -37.5, 2.0**20):
        ys = orc.softmax(x + c)
        assert np.array_equal(ys, y), c


def check_softmax_constant_row(orc):
    for n in (1, 2, 3, 64, 1000, 4096):
        y = orc.softmax(np.full((1, n), 1.25))
        assert np.allclose(y, 1.0 / n, rtol=2e-16, atol=0), n
    y = orc.softmax(np.array([[5.0]]))
    assert y[0, 0] == 1.0


def check_softmax_two_elements(orc):
    for a, b in [(0.0, 0.0), (1.0, -2.0), (-30.0, 5.0), (1000.0, 999.0), (0.5, 40.0)]:
        y = orc.softmax(np.array([[a, b]]))
        ra = 1.0 / (1.0 + math.exp(b - a))
        rb = 1.0 / (1.0 + math.exp(a - b))
        assert _rel(y[0], [ra, rb]) <= 1e-15, (a, b, y)


def check_softmax_brute_force(orc):
    import mpmath

    mpmath.mp.dps = 50
    r = _rng(11)
    for n in (1, 2, 3, 5, 8, 13, 16):
        for scale in (1.0, 10.0):
            x = scale * r.standard_normal(n)
            y = orc.softmax(x[None, :])[0]
            ex = [mpmath.exp(mpmath.mpf(float(v))) for v in x]
            s = mpmath.fsum(ex)
            ref = np.array([float(e / s) for e in ex])
            assert _rel(y, ref) <= 4e-15, (n, scale)


def check_softmax_torch(orc):
    import torch

    x = 6.0 * _rng(5).standard_normal((16, 1000))
    x[::4] += 1000.0
    y = orc.softmax(x)
    ref = torch.softmax(torch.from_numpy(x), dim=1).numpy()
    assert _rel(y, ref) <= 1e-13


# ----------------------------------------------------------- online / split


def check_online_stats_match_definition(orc):
    for n in (1, 5, 1000, 4099, 262144):
        x = 3.0 * _rng(n + 1).standard_normal(n)
        m0, d0 = orc.softmax_stats(x)
        for block in sorted({1, 3, 4096, n, n + 5}):
            if n >= 100000 and block < 64:
                continue  # keep the CPU suite short
            m, d = orc.online_stats(x, block)
            assert m == m0, (n, block)
            assert abs(d - d0) <= 1e-12 * d0, (n, block, d, d0)


def check_online_geometric_rows(orc):
    # x_j = -a j: max 0, d = (1 - q^N) / (1 - q) with q = e^-a; every block
    # starts below the running max.  x_j = +a j: max (N-1) a and the running
    # max rises in every block, so each step rescales the old sum.
    a = 0.01
    for n in (1000, 4099):
        q = math.exp(-a)
        dgeo = (1.0 - q**n) / (1.0 - q)
        j = np.arange(n, dtype=np.float64)
        for block in (1, 7, 64, n):
            m, d = orc.online_stats(-a * j, block)
            assert m == 0.0 and abs(d - dgeo) <= 1e-13 * dgeo, (n, block, d, dgeo)
            m, d = orc.online_stats(a * j, block)
            assert m == a * (n - 1), (n, block)
            assert abs(d - dgeo) <= 1e-12 * dgeo, (n, block, d, dgeo)


def check_merge_algebra(orc):
    ident = (-math.inf, 0.0)
    for s in [(0.5, 3.0), (-2.0, 1.0), (1000.0, 7.5)]:
        assert orc.merge(ident, s) == s and orc.merge(s, ident) == s
    assert orc.merge(ident, ident) == ident
    r = _rng(21)
    for _ in range(20):
        a, b, c = [(float(r.normal() * 5), float(r.uniform(1, 100))) for _ in range(3)]
        assert orc.merge(a, b) == orc.merge(b, a)
        l = orc.merge(orc.merge(a, b), c)
        rr = orc.merge(a, orc.merge(b, c))
        assert l[0] == rr[0] and abs(l[1] - rr[1]) <= 1e-15 * abs(l[1])
    # merging the two halves of a row gives the whole row's statistics
    x = 3.0 * r.standard_normal(1001)
    for cut in (1, 500, 1000):
        m, d = orc.merge(orc.softmax_stats(x[:cut]), orc.softmax_stats(x[cut:]))
        m0, d0 = orc.softmax_stats(x)
        assert m == m0 and abs(d - d0) <= 1e-14 * d0, cut
    # the merged sum is rescaled to the larger max: (0, 1) + (ln 2, 1) -> (ln 2, 1.5)
    m, d = orc.merge((0.0, 1.0), (math.log(2.0), 1.0))
    assert m == math.log(2.0) and abs(d - 1.5) <= 4e-16


def check_split_stats_match_definition(orc):
    for n in (5, 1000, 262144):
        x = 3.0 * _rng(n + 2).standard_normal(n)
        m0, d0 = orc.softmax_stats(x)
        for S in (1, 2, 3, 64, n, n + 3):
            if S > 4096:
                continue
            m, d, mp, dp = orc.split_stats(x, S)
            assert m == m0 and abs(d - d0) <= 1e-13 * d0, (n, S)
            C = -(-n // S)
            for s in range(S):
                chunk = x[s * C:min(n, (s + 1) * C)]
                if chunk.size == 0:
                    assert mp[s] == -math.inf and dp[s] == 0.0
                else:
                    assert mp[s] == chunk.max(), (n, S, s)


def check_online_and_split_outputs(orc):
    x = 3.0 * _rng(9).standard_normal((4, 4099))
    y0 = orc.softmax(x)
    for block in (1, 64, 4099):
        assert _rel(orc.online_softmax(x, block), y0) <= 1e-13, block
    for S in (1, 2, 64, 4099):
        assert _rel(orc.split_softmax(x, S), y0) <= 1e-13, S


def check_softmax_apply(orc):
    # the output pass with a row's own statistics gives that row's softmax at
    # any subset of its columns (torch.softmax in float64)
    import torch

    x = 5.0 * _rng(43).standard_normal(3001)
    m, d = orc.softmax_stats(x)
    cols = np.array([0, 7, 1500, 2999, 3000])
    ref = torch.softmax(torch.from_numpy(x), dim=0).numpy()[cols]
    assert _rel(orc.softmax_apply(x[cols], m, d), ref) <= 1e-13


def check_neg_inf_parts(orc):
    # A value of -inf adds exp(-inf - m) = 0 to the sum of any part with a
    # finite max m, so a row's (max, sum) are those of its finite values
    # alone; a part (block or chunk) holding only -inf has the empty part's
    # state (-inf, 0), the start state of the recurrence ("第 6 讲" §7.2), and
    # must not turn the merge into NaN.  References: numpy's max and an fsum of
    # exp(x - max) over the finite values; torch.softmax in float64, which
    # gives exact zeros at -inf inputs.
    import torch

    n = 4099
    base = 3.0 * _rng(41).standard_normal(n)

    def expect(row):
        fin = row[np.isfinite(row)]
        m = float(fin.max())
        return m, math.fsum(np.exp(fin - m).tolist())

    def same(got, want, what):
        assert got[0] == want[0], (what, got, want)
        assert abs(got[1] - want[1]) <= 1e-13 * want[1], (what, got, want)

    rows = []
    for k in (1, 3, 64, 1025, n - 1):  # -inf over the first k values
        r = base.copy()
        r[:k] = -math.inf
        rows.append((f"lead{k}", r))
    for S in (2, 3, 64):
        C = -(-n // S)
        for s in (0, S // 2, S - 1):  # chunk s all -inf, the others finite
            r = base.copy()
            r[s * C:min(n, (s + 1) * C)] = -math.inf
            rows.append((f"S{S}c{s}", r))
    r = base.copy()
    r[::5] = -math.inf  # scattered -inf in every block
    rows.append(("every5", r))
    for what, r in rows:
        want = expect(r)
        same(orc.softmax_stats(r), want, what)
        for block in (1, 3, 64, 4096, n):
            same(orc.online_stats(r, block), want, (what, block))
        for S in (2, 3, 64, n):
            m, d, mp, dp = orc.split_stats(r, S)
            same((m, d), want, (what, S))
            assert not np.any(np.isnan(dp)), (what, S)
        ref = torch.softmax(torch.from_numpy(r[None, :]), dim=1).numpy()
        zero = ~np.isfinite(r)
        for y in (orc.softmax(r[None, :]), orc.online_softmax(r[None, :], 64),
                  orc.online_softmax(r[None, :], 1), orc.split_softmax(r[None, :], 3),
                  orc.split_softmax(r[None, :], 64)):
            assert np.all(y[0, zero] == 0.0), what
            assert _rel(y[0, ~zero], ref[0, ~zero]) <= 1e-13, what
    # every value -inf: (-inf, 0) for every part and for the row; the
    # normalised row is 0/0 = NaN, as the plain definition gives
    r = np.full(n, -math.inf)
    assert orc.softmax_stats(r) == (-math.inf, 0.0)
    for block in (1, 3, n):
        assert orc.online_stats(r, block) == (-math.inf, 0.0), block
    for S in (2, 3, 64):
        m, d, mp, dp = orc.split_stats(r, S)
        assert (m, d) == (-math.inf, 0.0) and np.all(dp == 0.0), S
    for y in (orc.softmax(r[None, :]), orc.online_softmax(r[None, :], 3),
              orc.split_softmax(r[None, :], 64)):
        assert np.all(np.isnan(y))


# ---------------------------------------------------------------- GeLU


def check_gelu_basic(orc):
    z = np.array([0.0, 1e-30, -1e-30])
    y = orc.gelu_tanh(z)
    assert y[0] == 0.0 and abs(y[1] - 0.5e-30) <= 1e-45
    zz = np.linspace(-12.0, 12.0, 4801)
    diff = orc.gelu_tanh(zz) - orc.gelu_tanh(-zz)
    assert np.all(np.abs(diff - zz) <= 4e-16 * np.maximum(np.abs(zz), 1.0))
    big = np.array([10.0, 20.0, 40.0])
    assert np.all(np.abs(orc.gelu_tanh(big) - big) <= 1e-15 * big)
    neg = orc.gelu_tanh(-big)
    assert np.all(neg <= 0.0) and np.all(neg > -1e-30)


def check_gelu_torch(orc):
    import torch

    z = np.concatenate([np.linspace(-15, 15, 30001), 5.0 * _rng(4).standard_normal(1000)])
    y = orc.gelu_tanh(z)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    # 1 + tanh(u) cancels for z << 0 in both evaluations: absolute 1e-15 there
    assert np.all(np.abs(y - ref) <= 1e-15 * np.maximum(np.abs(ref), 1.0))
    pos = z > 0
    assert np.all(np.abs(y[pos] - ref[pos]) <= 1e-15 * np.abs(ref[pos]))


def check_gelu_not_erf(orc):
    z = np.linspace(-6, 6, 120001)
    y = orc.gelu_tanh(z)
    erf = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in z])
    gap = np.abs(y - erf)
    k = int(gap.argmax())
    assert 4.6e-4 <= gap[k] <= 4.8e-4 and -2.8 <= z[k] <= -2.6, (gap[k], z[k])


# ------------------------------------------------------------- LayerNorm


def check_layernorm_normalized_moments(orc):
    r = _rng(31)
    for n in (2, 3, 768, 1000, 4096):
        x = r.standard_normal((3, n)) * np.array([[1.0], [0.003], [50.0]]) + np.array(
            [[0.0], [1.25], [-7.0]])
        xh = orc.layernorm_normalize(x, EPS)
        for i in range(3):
            s2 = np.var(x[i])
            # rounding of x - mean is relative to |x|, magnified by rstd
            scale = 1e-15 * np.abs(x[i]).max() / math.sqrt(s2 + EPS)
            assert abs(xh[i].mean()) <= scale, (n, i)
            assert abs(np.mean(xh[i] ** 2) - s2 / (s2 + EPS)) <= 4 * scale, (n, i)


def check_layernorm_torch(orc):
    import torch
    import torch.nn.functional as F

    r = _rng(33)
    n = 768
    x = r.standard_normal((8, n))
    x[3] = 1.25 + 3e-3 * r.standard_normal(n)  # variance ~ eps
    w = 1.0 + 0.1 * r.standard_normal(n)
    b = 0.1 * r.standard_normal(n)
    xt = torch.from_numpy(x)
    for ww, bb in [(np.ones(n), np.zeros(n)), (w, b)]:
        y = orc.layernorm_gelu(x, ww, bb, EPS)
        ln = F.layer_norm(xt, (n,), torch.from_numpy(ww), torch.from_numpy(bb), EPS)
        ref = F.gelu(ln, approximate="tanh").numpy()
        assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1.0)) <= 1e-13


def check_layernorm_constant_row(orc):
    import torch
    import torch.nn.functional as F

    n = 768
    b = 0.1 * _rng(35).standard_normal(n)
    w = 1.0 + 0.1 * _rng(36).standard_normal(n)
    y = orc.layernorm_gelu(np.full((1, n), 1.25), w, b, EPS)[0]
    # x_hat is exactly 0, so z is exactly b: bitwise GeLU(b)
    assert np.array_equal(y, orc.gelu_tanh(b))
    ref = F.gelu(torch.from_numpy(b), approximate="tanh").numpy()
    assert np.all(np.abs(y - ref) <= 1e-15 * np.abs(ref))
    y1 = orc.layernorm_gelu(np.array([[3.0]]), np.array([2.0]), np.array([0.5]), EPS)
    assert abs(y1[0, 0] - F.gelu(torch.tensor(0.5, dtype=torch.float64),
                                 approximate="tanh").item()) <= 1e-16


def check_layernorm_eps_placement(orc):
    # Variance ~ eps: rstd is 1 / sqrt(var + eps), and the biased (divide by N)
    # variance is used.  Compare with numpy's population variance.
    x = 1.25 + 3e-3 * _rng(37).standard_normal(768)
    mean, var, rstd = orc.layernorm_stats(x, EPS)
    assert abs(mean - np.mean(x)) <= 1e-15
    assert abs(var - np.var(x)) <= 1e-15 * np.var(x) + 1e-22
    assert abs(rstd - 1.0 / math.sqrt(np.var(x) + EPS)) <= 1e-13 * rstd
    # the eps-less value differs at O(1) on this row
    assert abs(rstd * math.sqrt(np.var(x)) - 1.0) > 0.2


# --------------------------------------------------------------- RMSNorm


def check_rmsnorm_torch(orc):
    import torch
    import torch.nn.functional as F

    r = _rng(41)
    for n in (1, 7, 768, 4096):
        x = r.standard_normal((6, n)) * np.array([[1.0], [1e-3], [30.0], [1.0], [5.0], [0.1]])
        x[3] += 2.5  # rows with a mean: RMSNorm does not centre
        w = 1.0 + 0.1 * r.standard_normal(n)
        y = orc.rmsnorm(x, w, EPS)
        ref = F.rms_norm(torch.from_numpy(x), (n,), torch.from_numpy(w), EPS).numpy()
        assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1.0)) <= 1e-14, n


def check_rmsnorm_invariants(orc):
    r = _rng(43)
    n = 1000
    x = r.standard_normal((4, n)) * np.array([[1.0], [1e-3], [8.0], [0.02]]) + np.array(
        [[0.0], [0.0], [3.0], [0.0]])
    w = 1.0 + 0.1 * r.standard_normal(n)
    y = orc.rmsnorm(x, w, EPS)
    for i in range(4):
        ms = np.mean(x[i] ** 2)
        assert abs(np.mean((y[i] / w) ** 2) - ms / (ms + EPS)) <= 1e-13
    assert np.array_equal(orc.rmsnorm(-x, w, EPS), -y)
    # constant row c: y = c / sqrt(c^2 + eps) w
    c = 0.75
    yc = orc.rmsnorm(np.full((1, n), c), w, EPS)[0]
    assert np.all(np.abs(yc - c / math.sqrt(c * c + EPS) * w) <= 1e-15 * np.abs(w) + 1e-16)
    # eps-sensitive row: mean square ~ eps
    xe = 3e-3 * r.standard_normal(n)
    ms, inv = orc.rms_stats(xe, EPS)
    assert abs(ms - np.mean(xe * xe)) <= 1e-15 * ms
    assert abs(inv - 1.0 / math.sqrt(np.mean(xe * xe) + EPS)) <= 1e-13 * inv
    assert abs(inv * math.sqrt(ms) - 1.0) > 0.2


def check_residual_rmsnorm(orc):
    import torch
    import torch.nn.functional as F

    r = _rng(47)
    n = 768
    x = np.float32(1.0) * r.standard_normal((5, n)).astype(np.float32)
    res = (3.0 * r.standard_normal((5, n))).astype(np.float32)
    w = (1.0 + 0.1 * r.standard_normal(n)).astype(np.float32)
    y, ro = orc.residual_rmsnorm(x, res, w, EPS)
    # the sum of two fp32 values is exact in double
    assert np.array_equal(ro, x.astype(np.float64) + res.astype(np.float64))
    ref = F.rms_norm(torch.from_numpy(ro), (n,), torch.from_numpy(w.astype(np.float64)),
                     EPS).numpy()
    assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1.0)) <= 1e-14
    # residual of zero: plain RMSNorm of x
    y0, ro0 = orc.residual_rmsnorm(x, np.zeros_like(x), w, EPS)
    assert np.array_equal(ro0, x.astype(np.float64))
    assert np.array_equal(y0, orc.rmsnorm(x, w, EPS))


# ------------------------------------------------------------ exact GeLU


def check_gelu_erf_basic(orc):
    z = np.linspace(-12.0, 12.0, 2401)
    y = orc.gelu_erf(z)
    assert orc.gelu_erf(np.array([0.0]))[0] == 0.0
    # erf is odd: GeLU(z) - GeLU(-z) = z
    assert np.max(np.abs((y - orc.gelu_erf(-z)) - z) / np.maximum(np.abs(z), 1e-300)) <= 4e-16
    assert np.all(np.abs(y[z >= 9.0] - z[z >= 9.0]) <= 1e-15 * z[z >= 9.0])
    assert np.all(np.abs(y[z <= -9.0]) <= 1e-17)


def check_gelu_erf_brute_force(orc):
    import mpmath

    mpmath.mp.dps = 50
    z = np.array([-6.0, -3.5, -2.7, -1.0, -0.25, 1e-3, 0.5, 1.0, 2.0, 4.75])
    y = orc.gelu_erf(z)
    ref = np.array([float(mpmath.mpf(float(v)) * mpmath.ncdf(mpmath.mpf(float(v)))) for v in z])
    # relative where 1 + erf does not cancel; in the negative tail the literal
    # form is accurate to ~1e-16 absolute (the unit scale of the comparisons)
    ok = z >= -1.0
    assert _rel(y[ok], ref[ok]) <= 2e-15
    assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1.0)) <= 2e-15


def check_gelu_erf_torch_and_tanh_gap(orc):
    import torch
    import torch.nn.functional as F

    z = np.linspace(-8.0, 8.0, 16001)
    y = orc.gelu_erf(z)
    ref = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1.0)) <= 1e-15
    gap = np.abs(y - orc.gelu_tanh(z))
    k = int(np.argmax(gap))
    assert 4.70e-4 <= gap[k] <= 4.76e-4 and abs(z[k] + 2.70) <= 0.02, (gap[k], z[k])


# ------------------------------------------------- split LayerNorm statistics


def check_chunk_moments_closed_form(orc):
    for n, a, d in [(1, 3.5, 0.0), (2, -1.0, 2.0), (10, 0.0, 1.0), (1001, 7.25, -0.125),
                    (65536, -3.0, 2.0**-10)]:
        x = a + d * np.arange(n, dtype=np.float64)
        mean, m2 = orc.chunk_moments(x)
        assert abs(mean - (a + d * (n - 1) / 2.0)) <= 1e-15 * max(abs(a), 1.0) * 4, (n, mean)
        ref = d * d * n * (n * n - 1) / 12.0
        assert abs(m2 - ref) <= 1e-13 * max(ref, 1e-300), (n, m2, ref)
    # a constant whose partial sums are exact: mean exactly c, M2 exactly 0
    mean, m2 = orc.chunk_moments(np.full(777, 0.375))
    assert mean == 0.375 and m2 == 0.0


def check_chan_merge_algebra(orc):
    r = _rng(53)
    x = 5.0 + 2.0 * r.standard_normal(1000)
    whole = orc.chunk_moments(x)
    for cut in (1, 2, 333, 500, 999):
        a = (cut, *orc.chunk_moments(x[:cut]))
        b = (1000 - cut, *orc.chunk_moments(x[cut:]))
        n, mean, m2 = orc.chan_merge(a, b)
        assert n == 1000
        assert abs(mean - whole[0]) <= 1e-14 * abs(whole[0]), cut
        assert abs(m2 - whole[1]) <= 1e-13 * whole[1], cut
        n2, mean2, m22 = orc.chan_merge(b, a)  # commutative (up to rounding)
        assert abs(mean2 - mean) <= 1e-14 * abs(mean) and abs(m22 - m2) <= 1e-13 * m2
    e = (0.0, 0.0, 0.0)
    s = (17.0, 1.5, 4.25)
    assert orc.chan_merge(e, s) == s and orc.chan_merge(s, e) == s
    # two single points: mean (a+b)/2, M2 = (a-b)^2/2
    n, mean, m2 = orc.chan_merge((1.0, 3.0, 0.0), (1.0, -1.0, 0.0))
    assert (n, mean, m2) == (2.0, 1.0, 8.0)
    # associativity over three pieces
    p = [(k, *orc.chunk_moments(x[i:i + k])) for i, k in ((0, 100), (100, 650), (750, 250))]
    left = orc.chan_merge(orc.chan_merge(p[0], p[1]), p[2])
    right = orc.chan_merge(p[0], orc.chan_merge(p[1], p[2]))
    assert abs(left[1] - right[1]) <= 1e-14 * abs(left[1])
    assert abs(left[2] - right[2]) <= 1e-13 * left[2]
    # arithmetic progression halves merge to the closed form
    ap = np.arange(64, dtype=np.float64)
    n, mean, m2 = orc.chan_merge((32.0, *orc.chunk_moments(ap[:32])),
                                 (32.0, *orc.chunk_moments(ap[32:])))
    assert mean == 31.5 and abs(m2 - 64 * (64 * 64 - 1) / 12.0) <= 1e-12


def check_split_moments_match_whole_row(orc):
    r = _rng(59)
    for n in (1, 5, 768, 4099, 262144):
        x = -2.0 + 3.0 * r.standard_normal(n)
        mean, m2 = orc.chunk_moments(x)
        for S in sorted({1, 2, 3, 7, 64, n, n + 3}):
            sm, sm2, npart, mpart, m2part = orc.split_moments(x, S)
            assert abs(sm - mean) <= 1e-13 * max(abs(mean), 1.0), (n, S)
            assert abs(sm2 - m2) <= 1e-12 * max(m2, 1e-300), (n, S, sm2, m2)
            assert npart.sum() == n and np.all(npart >= 0)
            C = -(-n // S)
            for s in (0, S // 2, S - 1):
                lo, hi = s * C, min(n, (s + 1) * C)
                if hi > lo:
                    cm, cm2 = orc.chunk_moments(x[lo:hi])
                    assert npart[s] == hi - lo and mpart[s] == cm and m2part[s] == cm2
                else:
                    assert npart[s] == 0


def check_layernorm_gelu_ex(orc):
    import torch
    import torch.nn.functional as F

    r = _rng(61)
    n = 3000
    x = r.standard_normal((5, n)) * np.array([[1.0], [10.0], [1e-3], [1.0], [4.0]])
    x[3] += 100.0  # a large mean: the split statistics must still centre
    w = 1.0 + 0.1 * r.standard_normal(n)
    b = 0.1 * r.standard_normal(n)
    base = orc.layernorm_gelu(x, w, b, EPS)
    assert np.array_equal(orc.layernorm_gelu_ex(x, w, b, EPS, "tanh", 0), base)
    for S in (1, 5, 64, n + 1):
        y = orc.layernorm_gelu_ex(x, w, b, EPS, "tanh", S)
        assert np.max(np.abs(y - base) / np.maximum(np.abs(base), 1.0)) <= 1e-13, S
    xt = torch.from_numpy(x)
    ln = F.layer_norm(xt, (n,), torch.from_numpy(w), torch.from_numpy(b), EPS)
    ref = F.gelu(ln, approximate="none").numpy()
    for S in (0, 7):
        y = orc.layernorm_gelu_ex(x, w, b, EPS, "erf", S)
        assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1.0)) <= 1e-13, S
    assert np.max(np.abs(orc.layernorm_gelu_ex(x, w, b, EPS, "erf", 0) - base)) > 1e-4
    # no activation: the LayerNorm alone ([TKE] §4.1) is F.layer_norm, whole-row
    # and split statistics; a constant row gives exactly the bias
    ln = ln.numpy()
    for S in (0, 7):
        y = orc.layernorm_gelu_ex(x, w, b, EPS, "none", S)
        assert np.max(np.abs(y - ln) / np.maximum(np.abs(ln), 1.0)) <= 1e-13, S
    c = np.full((1, n), 3.25)
    assert np.array_equal(orc.layernorm_gelu_ex(c, w, b, EPS, "none", 0)[0], b)


# ------------------------------------------------------ row sum and max


def check_row_sum(orc):
    r = _rng(83)
    for n in (1, 2, 7, 1000, 262144):
        x = r.standard_normal((3, n)) * np.array([[1.0], [1e3], [1e-3]])
        s = orc.row_sum(x)
        for i in range(3):
            ref = math.fsum(x[i])
            assert abs(s[i] - ref) <= 1e-15 * np.abs(x[i]).sum() + 1e-300, (n, i)
    for n in (1, 10, 4097):
        ap = np.arange(n, dtype=np.float64)
        assert orc.row_sum(ap)[0] == n * (n - 1) / 2
    x = np.concatenate([np.full(500, 0.25), np.full(500, -0.25)])[None, :]
    assert orc.row_sum(x)[0] == 0.0
    assert orc.row_sum(np.array([[3.5]]))[0] == 3.5


def check_row_max(orc):
    r = _rng(89)
    for n in (1, 3, 1000, 65537):
        x = 5.0 * r.standard_normal((4, n))
        m = orc.row_max(x)
        assert np.array_equal(m, x.max(axis=1)), n
        perm = r.permutation(n)
        assert np.array_equal(orc.row_max(x[:, perm]), m)
    x = r.standard_normal((3, 100))
    x[0, 50] = np.nan
    x[1, :] = -np.inf
    x[2, 99] = np.inf
    m = orc.row_max(x)
    assert np.isnan(m[0]) and m[1] == -np.inf and m[2] == np.inf


# ------------------------------------------------------------- attention


def _sdpa(q, k, v, causal, scale=None):
    import torch
    import torch.nn.functional as F

    t = [torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v)]
    return F.scaled_dot_product_attention(*t, is_causal=causal, scale=scale).numpy()


def check_attention_torch(orc):
    r = _rng(107)
    for T, d in ((1, 8), (7, 16), (64, 64), (130, 128)):
        q, k, v = (r.standard_normal((2, 3, T, d)) for _ in range(3))
        for causal in (False, True):
            o = orc.attention(q, k, v, causal)
            ref = _sdpa(q, k, v, causal)
            assert np.max(np.abs(o - ref)) <= 1e-13, (T, d, causal)
    q, k, v = (3.0 * r.standard_normal((1, 2, 33, 32)) for _ in range(3))
    o = orc.attention(q, k, v, True, scale=0.3)
    assert np.max(np.abs(o - _sdpa(q, k, v, True, 0.3))) <= 1e-13


def check_attention_closed_forms(orc):
    r = _rng(109)
    T, d = 40, 16
    q, k = r.standard_normal((1, T, d)), r.standard_normal((1, T, d))
    c = r.standard_normal(d)
    v = np.tile(c, (1, T, 1))
    for causal in (False, True):
        assert np.max(np.abs(orc.attention(q, k, v, causal) - c)) <= 1e-14
    v = r.standard_normal((1, T, d))
    z = np.zeros((1, T, d))
    o = orc.attention(z, k, v, False)
    assert np.max(np.abs(o[0] - v[0].mean(axis=0))) <= 1e-14
    o = orc.attention(z, k, v, True)
    prefix = np.cumsum(v[0], axis=0) / np.arange(1, T + 1)[:, None]
    assert np.max(np.abs(o[0] - prefix)) <= 1e-14
    o = orc.attention(q, k, v, True)
    assert np.array_equal(o[0, 0], v[0, 0])
    o1 = orc.attention(q[:, :1], k[:, :1], v[:, :1], False)
    assert np.array_equal(o1, v[:, :1])
    # a dominant score: query 5 aligned with key 11 at large scale
    qd = np.zeros((1, T, d))
    kd = 0.01 * r.standard_normal((1, T, d))
    qd[0, 5, 0] = 1.0
    kd[0, 11, 0] = 1.0
    o = orc.attention(qd, kd, v, False, scale=200.0)
    assert np.max(np.abs(o[0, 5] - v[0, 11])) <= 1e-12


def check_attention_large_scores(orc):
    # scores in the thousands: exp without the max shift overflows
    r = _rng(137)
    q, k, v = (r.standard_normal((1, 2, 48, 16)) for _ in range(3))
    for causal in (False, True):
        o = orc.attention(q, k, v, causal, scale=500.0)
        assert np.all(np.isfinite(o))
        assert np.max(np.abs(o - _sdpa(q, k, v, causal, 500.0))) <= 1e-12, causal


def check_attention_permutation(orc):
    r = _rng(113)
    q, k, v = (r.standard_normal((2, 50, 8)) for _ in range(3))
    perm = r.permutation(50)
    o = orc.attention(q, k, v, False)
    op = orc.attention(q, k[:, perm], v[:, perm], False)
    assert np.max(np.abs(o - op)) <= 1e-14
    # a permutation of keys changes the causal result (the mask is positional)
    assert np.max(np.abs(orc.attention(q, k, v, True) - orc.attention(q, k[:, perm], v[:, perm],
                                                                      True))) > 1e-3


def check_attention_brute_force(orc):
    import mpmath

    mpmath.mp.dps = 50
    r = _rng(127)
    for T, d, causal in ((3, 2, False), (4, 3, True), (5, 1, True)):
        q, k, v = (2.0 * r.standard_normal((1, T, d)) for _ in range(3))
        o = orc.attention(q, k, v, causal)
        sc = mpmath.mpf(1) / mpmath.sqrt(d)
        for i in range(T):
            n = i + 1 if causal else T
            w = [mpmath.exp(sc * mpmath.fsum(mpmath.mpf(float(q[0, i, c])) * float(k[0, j, c])
                                             for c in range(d))) for j in range(n)]
            den = mpmath.fsum(w)
            for c in range(d):
                ref = mpmath.fsum(w[j] * float(v[0, j, c]) for j in range(n)) / den
                assert abs(o[0, i, c] - float(ref)) <= 4e-15 * max(1.0, abs(float(ref)))


def check_attention_rows(orc):
    # selected query rows at their positions equal torch's attention in
    # float64 at those rows (causal and not), and the first causal row sees
    # only key 0
    import torch

    r = _rng(71)
    T, d = 97, 16
    q, k, v = (r.standard_normal((T, d)) for _ in range(3))
    pos = np.array([0, 1, 5, 48, 95, 96])
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[None]), torch.from_numpy(k[None]), torch.from_numpy(v[None]),
            is_causal=causal).numpy()[0]
        o = orc.attention_rows(q[pos], pos, k, v, causal)
        assert np.max(np.abs(o - ref[pos])) <= 1e-13, causal
    o = orc.attention_rows(q[:1], [0], k, v, True)
    assert np.array_equal(o[0], v[0])


def check_flash_attention_tiled(orc):
    r = _rng(131)
    for T, d in ((1, 4), (37, 16), (100, 32)):
        q, k, v = (2.0 * r.standard_normal((2, T, d)) for _ in range(3))
        for causal in (False, True):
            ref = orc.attention(q, k, v, causal)
            for br, bc in ((1, 1), (3, 5), (16, 16), (T, T), (T + 5, 7), (64, 3)):
                o = orc.flash_attention(q, k, v, causal, block_q=br, block_kv=bc)
                assert np.max(np.abs(o - ref)) <= 1e-13, (T, causal, br, bc)


PINS = [
    check_softmax_sums_to_one,
    check_softmax_shift_invariance,
    check_softmax_constant_row,
    check_softmax_two_elements,
    check_softmax_brute_force,
    check_softmax_torch,
    check_online_stats_match_definition,
    check_online_geometric_rows,
    check_merge_algebra,
    check_split_stats_match_definition,
    check_online_and_split_outputs,
    check_neg_inf_parts,
    check_softmax_apply,
    check_gelu_basic,
    check_gelu_torch,
    check_gelu_not_erf,
    check_layernorm_normalized_moments,
    check_layernorm_torch,
    check_layernorm_constant_row,
    check_layernorm_eps_placement,
    check_rmsnorm_torch,
    check_rmsnorm_invariants,
    check_residual_rmsnorm,
    check_gelu_erf_basic,
    check_gelu_erf_brute_force,
    check_gelu_erf_torch_and_tanh_gap,
    check_chunk_moments_closed_form,
    check_chan_merge_algebra,
    check_split_moments_match_whole_row,
    check_layernorm_gelu_ex,
    check_row_sum,
    check_row_max,
    check_attention_torch,
    check_attention_closed_forms,
    check_attention_large_scores,
    check_attention_permutation,
    check_attention_brute_force,
    check_flash_attention_tiled,
    check_attention_rows,
]
