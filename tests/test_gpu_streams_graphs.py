"""The C ABI under HIP graph capture and from several host threads and
streams: results must equal the eager single-stream results bit for bit
(every kernel here is deterministic)."""
import threading

import numpy as np
import pytest
import torch

import row_wise_amd as rk
import rowgen

pytestmark = pytest.mark.gpu
DEV = "cuda"
EPS = float(np.float32(1e-5))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rk.load()
    yield
    torch.cuda.synchronize()


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_graph_capture_and_replay():
    d = rowgen.make("ln_gelu_f32_4096x768")
    x = d["x"].to(DEV)
    w, b = d["w"].to(DEV), d["b"].to(DEV)
    xs = rowgen.randn(64, 20000, seed=301).to(DEV)
    res = rowgen.residual("ln_gelu_f32_4096x768").to(DEV)
    q, k, v = (t.to(DEV) for t in rowgen.attention_qkv(1, 4, 300, 128, torch.bfloat16, seed=302))
    ws = torch.empty(rk.rk_online_softmax_workspace_bytes(64, 20000, 4, rk.RK_F32),
                     dtype=torch.uint8, device=DEV)
    # 8 rows of 65536: rk_softmax and rk_layernorm_gelu split them with the
    # partials kept in the output (three kernels, no workspace)
    xl = rowgen.randn(8, 65536, seed=303).to(DEV)
    wl, bl = (t.to(DEV) for t in rowgen.ln_params(65536, torch.Generator().manual_seed(304),
                                                  torch.float32))
    # bf16 rows of 8192: the persistent LayerNorm kernel, both GeLU forms
    xp = rowgen.randn(300, 8192, seed=305).to(torch.bfloat16).to(DEV)
    wp, bp = (t.to(DEV) for t in rowgen.ln_params(8192, torch.Generator().manual_seed(306),
                                                  torch.bfloat16))
    wsr = torch.empty(rk.rk_row_reduce_workspace_bytes(64, 20000, 8, rk.RK_F32),
                      dtype=torch.uint8, device=DEV)
    outs = {n: None for n in ("ln", "sm", "rms", "ro", "attn", "sml", "lnl", "lnp", "lnpe",
                              "rs", "rm")}

    def step():
        outs["ln"] = rk.rk_layernorm_gelu(x, w, b, EPS, out=outs["ln"])
        outs["sm"] = rk.rk_online_softmax(xs, num_splits=4, out=outs["sm"], workspace=ws)
        outs["sml"] = rk.rk_softmax(xl, out=outs["sml"])
        outs["lnl"] = rk.rk_layernorm_gelu(xl, wl, bl, EPS, out=outs["lnl"])
        y, r = rk.rk_residual_rmsnorm(x, res, w, EPS, out=outs["rms"], residual_out=outs["ro"])
        outs["rms"], outs["ro"] = y, r
        outs["attn"] = rk.rk_flash_attention(q, k, v, causal=True, out=outs["attn"])
        outs["lnp"] = rk.rk_layernorm_gelu(xp, wp, bp, EPS, out=outs["lnp"])
        outs["lnpe"] = rk.rk_layernorm_gelu_ex(xp, wp, bp, EPS, gelu="erf", out=outs["lnpe"])
        # the split row sum and max on a preallocated workspace
        outs["rs"] = rk.rk_row_sum_ex(xs, num_splits=8, out=outs["rs"], workspace=wsr)
        outs["rm"] = rk.rk_row_max_ex(xs, num_splits=8, out=outs["rm"], workspace=wsr)

    step()  # allocates the outputs, eagerly
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        step()  # warm the side stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        # new inputs each time, written by eager work between replays
        x.copy_(rowgen.randn(4096, 768, seed=310 + rep).to(DEV))
        xs.copy_(rowgen.randn(64, 20000, seed=320 + rep).to(DEV))
        xl.copy_(rowgen.randn(8, 65536, seed=330 + rep).to(DEV))
        xp.copy_(rowgen.randn(300, 8192, seed=340 + rep).to(torch.bfloat16).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {n: t.clone() for n, t in outs.items()}
        step()  # eager, same buffers
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(bits(got[n]), bits(outs[n])), (rep, n)


def test_threads_and_streams():
    # fp32 rows of 1000-1111 (general tiles), and bf16 rows of 8192 (the
    # persistent LayerNorm kernel, whose per-device workgroup count is shared)
    inputs = [rowgen.randn(2048, 1000 + 37 * i, seed=400 + i).to(DEV) for i in range(4)]
    inputs += [rowgen.randn(700 + 9 * i, 8192, seed=410 + i).to(torch.bfloat16).to(DEV)
               for i in range(4)]
    ws = [torch.ones(x.shape[1], dtype=x.dtype, device=DEV) for x in inputs]
    bs = [torch.zeros(x.shape[1], dtype=x.dtype, device=DEV) for x in inputs]
    ref = [(rk.rk_softmax(x), rk.rk_layernorm_gelu(x, w, b, EPS))
           for x, w, b in zip(inputs, ws, bs)]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    a = rk.rk_softmax(inputs[i])
                    c = rk.rk_layernorm_gelu(inputs[i], ws[i], bs[i], EPS)
                s.synchronize()
                if not (torch.equal(bits(a), bits(ref[i][0])) and
                        torch.equal(bits(c), bits(ref[i][1]))):
                    errors.append(i)
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
