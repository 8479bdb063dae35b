"""The parity comparator: it accepts a faithful fp32 evaluation and rejects
planted mistakes of the size the kernels could plausibly make."""
import math

import numpy as np
import torch

import oracle
import rowgen
from tolerance import TOL, rel_err_floor1, rel_err_softmax

EPS = float(np.float32(1e-5))


def _softmax_f32(x):
    x = np.asarray(x, dtype=np.float32)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=1, keepdims=True)


def test_fp32_softmax_within_tolerance():
    d = rowgen.make("softmax_f32_8192x1000", rows=256)
    x = d["x_softmax"].numpy()
    assert rel_err_softmax(_softmax_f32(x), oracle.softmax(x)) <= TOL["f32"]


def test_missing_max_subtraction_is_rejected():
    d = rowgen.make("softmax_f32_8192x1000", rows=32)
    x = d["x_softmax"].numpy().astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        bad = e / e.sum(axis=1, keepdims=True)
    assert rel_err_softmax(bad, oracle.softmax(x)) > TOL["f32"]


def test_dropped_split_rescale_is_rejected():
    x = 3.0 * np.random.default_rng(0).standard_normal((2, 4096))
    ref = oracle.softmax(x)
    parts = x.reshape(2, 64, 64)
    m = parts.max(axis=2)
    d = np.exp(parts - m[..., None]).sum(axis=2)
    M = m.max(axis=1, keepdims=True)
    D = d.sum(axis=1, keepdims=True)  # rescale factor exp(m_s - M) dropped
    bad = np.exp(x - M) / D
    assert rel_err_softmax(bad, ref) > TOL["f32"]


def test_padded_variance_bug_is_rejected():
    # Variance taken over a power-of-two padded row (padding centred too),
    # the mistake the LayerNorm page warns about.
    d = rowgen.make("ln_gelu_f32_4096x768", rows=64)
    x, w, b = (d[k].numpy().astype(np.float64) for k in ("x", "w", "b"))
    N, BLOCK = x.shape[1], 1024
    mean = x.sum(axis=1, keepdims=True) / N
    var = (((x - mean) ** 2).sum(axis=1, keepdims=True) + (BLOCK - N) * mean**2) / N
    z = (x - mean) / np.sqrt(var + EPS) * w + b
    bad = oracle.gelu_tanh(z)
    ref = oracle.layernorm_gelu(x, w, b, EPS)
    assert rel_err_floor1(bad, ref) > TOL["f32"]


def test_erf_gelu_is_rejected():
    d = rowgen.make("ln_gelu_f32_4096x768", rows=64)
    x, w, b = (d[k] for k in ("x", "w", "b"))
    ln = torch.nn.functional.layer_norm(x.double(), (x.shape[1],), w.double(), b.double(), EPS)
    bad = torch.nn.functional.gelu(ln)  # exact erf form
    ref = oracle.layernorm_gelu(x, w, b, EPS)
    assert rel_err_floor1(bad, ref) > TOL["f32"]


def test_fp32_layernorm_gelu_within_tolerance():
    d = rowgen.make("ln_gelu_f32_4096x768", rows=128)
    x, w, b = (d[k] for k in ("x", "w", "b"))
    ln = torch.nn.functional.layer_norm(x, (x.shape[1],), w, b, EPS)
    y = torch.nn.functional.gelu(ln, approximate="tanh")
    ref = oracle.layernorm_gelu(x, w, b, EPS)
    assert rel_err_floor1(y, ref) <= TOL["f32"]


def test_nonfinite_is_rejected():
    ref = np.array([[0.25, 0.75]])
    assert rel_err_softmax(np.array([[math.nan, 0.75]]), ref) == math.inf
    assert rel_err_floor1(np.array([[math.inf, 0.75]]), ref) == math.inf
    assert rel_err_softmax(ref, ref) == 0.0


def test_pure_relative_above_threshold():
    from tolerance import rel_err_above

    ref = np.array([1e-4, -0.02, 0.5, 3.0])
    y = ref * np.array([1.5, 1.0 + 2e-6, 1.0 - 1e-6, 1.0])  # 50% off below the threshold
    assert rel_err_above(y, ref, 1e-2) <= 2.0001e-6
    assert rel_err_above(y, ref, 1e-5) >= 0.5
    assert rel_err_above(y, ref, 10.0) == 0.0
    assert rel_err_above(np.array([np.nan, 1.0]), np.array([1.0, 1.0]), 0.5) == float("inf")
    # an fp32 evaluation of config 2 holds 1e-5 as a pure relative error where |r| >= 0.01
    d = rowgen.make("ln_gelu_f32_4096x768", rows=128)
    x, w, b = (d[k].numpy().astype(np.float32) for k in ("x", "w", "b"))
    mean = x.mean(axis=1, keepdims=True, dtype=np.float32)
    var = ((x - mean) ** 2).mean(axis=1, keepdims=True, dtype=np.float32)
    z = ((x - mean) / np.sqrt(var + np.float32(EPS)) * w + b).astype(np.float32)
    k = np.float32(math.sqrt(2 / math.pi))
    y = (np.float32(0.5) * z * (np.float32(1) + np.tanh(k * (z + np.float32(0.044715) * z ** 3)))).astype(np.float32)
    ref = oracle.layernorm_gelu(x, w, b, EPS)
    assert rel_err_above(y, ref, 1e-2) <= TOL["f32"]
