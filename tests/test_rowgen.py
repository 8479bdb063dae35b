"""The seeded generators: same seed, same bytes; the recipes' structure."""
import torch

import rowgen


def test_deterministic():
    a = rowgen.make("tiny_f32_64x768")
    b = rowgen.make("tiny_f32_64x768")
    for k in ("x", "w", "b"):
        assert torch.equal(a[k], b[k])


def test_softmax_offsets():
    d = rowgen.make("softmax_f32_8192x1000", rows=64)
    x = d["x_softmax"]
    assert x.dtype == torch.float32 and x.shape == (64, 1000)
    means = x.mean(dim=1)
    assert torch.all(means[::16] > 990) and torch.all(means[1::16].abs() < 2)


def test_bf16_softmax_input_is_exact_multiple():
    d = rowgen.make("bf16_16384x4096", rows=8)
    assert d["x"].dtype == torch.bfloat16 and d["w"].dtype == torch.bfloat16
    assert torch.equal(d["x_softmax"].float(), 8.0 * d["x"].float())


def test_rows_prefix():
    full = rowgen.make("ln_gelu_f32_4096x768")
    part = rowgen.make("ln_gelu_f32_4096x768", rows=10)
    assert torch.equal(full["x"][:10], part["x"])
    assert torch.equal(full["w"], part["w"])


def test_residual_is_independent_and_seeded():
    d = rowgen.make("ln_gelu_f32_4096x768", rows=16)
    r = rowgen.residual("ln_gelu_f32_4096x768", rows=16)
    assert r.shape == d["x"].shape and r.dtype == d["x"].dtype
    assert torch.equal(r, rowgen.residual("ln_gelu_f32_4096x768")[:16])
    assert not torch.equal(r, d["x"])
    assert rowgen.residual("bf16_16384x4096", rows=2).dtype == torch.bfloat16
