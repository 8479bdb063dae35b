"""CPU oracle (double precision) -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``oracle/oracle.c``.  Only ``tests/``, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The HIP library (``row_wise_amd``) never imports it, and
the two share no code: the only thing both sides consume is the seeded input
generator in ``rowgen``.

All functions take array-likes (numpy or CPU torch tensors of any float
dtype), widen them exactly to float64, and return float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

__all__ = [
    "build", "Oracle", "default", "softmax", "softmax_stats", "online_softmax", "online_stats",
    "merge", "split_stats", "split_softmax", "gelu_tanh", "layernorm_stats", "layernorm_normalize",
    "layernorm_gelu", "rms_stats", "rmsnorm", "residual_rmsnorm", "gelu_erf", "chunk_moments",
    "chan_merge", "split_moments", "layernorm_gelu_ex", "row_sum", "row_max", "attention",
    "flash_attention",
]


def build(out: str = _LIB, src: str = _SRC) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _signatures():
    P = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    d = ctypes.c_double
    return {
        "oracle_softmax": [P, P, i64, i64],
        "oracle_softmax_stats": [P, i64, P, P],
        "oracle_online_stats": [P, i64, i64, P, P],
        "oracle_merge": [d, d, d, d, P, P],
        "oracle_split_stats": [P, i64, i64, P, P, P, P],
        "oracle_softmax_apply": [P, P, i64, d, d],
        "oracle_online_softmax": [P, P, i64, i64, i64],
        "oracle_split_softmax": [P, P, i64, i64, i64],
        "oracle_gelu_tanh_array": [P, P, i64],
        "oracle_layernorm_stats": [P, i64, d, P, P, P],
        "oracle_layernorm_normalize": [P, P, i64, i64, d],
        "oracle_layernorm_gelu": [P, P, P, P, i64, i64, d],
        "oracle_rms_stats": [P, i64, d, P, P],
        "oracle_rmsnorm": [P, P, P, i64, i64, d],
        "oracle_residual_rmsnorm": [P, P, P, P, P, i64, i64, d],
        "oracle_gelu_erf_array": [P, P, i64],
        "oracle_chunk_moments": [P, i64, P, P],
        "oracle_chan_merge": [d, d, d, d, d, d, P, P, P],
        "oracle_split_moments": [P, i64, i64, P, P, P, P, P],
        "oracle_layernorm_gelu_ex": [P, P, P, P, i64, i64, d, ctypes.c_int, i64],
        "oracle_row_sum": [P, P, i64, i64],
        "oracle_row_max": [P, P, i64, i64],
        "oracle_attention": [P, P, P, P, i64, i64, i64, ctypes.c_int, d],
        "oracle_flash_attention": [P, P, P, P, i64, i64, i64, ctypes.c_int, d, i64, i64],
        "oracle_attention_rows": [P, ctypes.POINTER(i64), i64, P, P, P, i64, i64, ctypes.c_int,
                                  d],
    }


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor (bf16 has no numpy dtype: widen in torch first)
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _rows(x):
    x = _f64(x)
    if x.ndim == 1:
        x = x[None, :]
    assert x.ndim == 2
    return x


class Oracle:
    """The oracle's functions, bound to one compiled copy of ``oracle.c``."""

    def __init__(self, lib_path: str = _LIB):
        if lib_path == _LIB and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(lib_path)
        for name, args in _signatures().items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = None
        self.lib = lib

    def softmax(self, x) -> np.ndarray:
        """Stable row softmax of a [M, N] array."""
        x = _rows(x)
        y = np.empty_like(x)
        self.lib.oracle_softmax(_p(x), _p(y), x.shape[0], x.shape[1])
        return y

    def softmax_stats(self, row):
        """(max, sum exp(x - max)) of one row."""
        r = _f64(row).ravel()
        m, d = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_softmax_stats(_p(r), r.size, ctypes.byref(m), ctypes.byref(d))
        return m.value, d.value

    def softmax_apply(self, values, m: float, d: float) -> np.ndarray:
        """exp(x - m) / d for the given values of a row whose statistics are
        (m, d): the output pass of the softmax, for sampled columns."""
        v = _f64(values).ravel()
        y = np.empty_like(v)
        self.lib.oracle_softmax_apply(_p(v), _p(y), v.size, float(m), float(d))
        return y

    def online_stats(self, row, block: int):
        """Streaming (m, d) of one row over blocks of ``block`` elements."""
        r = _f64(row).ravel()
        m, d = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_online_stats(_p(r), r.size, int(block), ctypes.byref(m), ctypes.byref(d))
        return m.value, d.value

    def merge(self, a, b):
        """Merge two partial states (m1, d1), (m2, d2)."""
        m, d = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_merge(float(a[0]), float(a[1]), float(b[0]), float(b[1]),
                              ctypes.byref(m), ctypes.byref(d))
        return m.value, d.value

    def split_stats(self, row, splits: int):
        """(m, d, m_parts, d_parts) of the split-row variant with ``splits`` chunks."""
        r = _f64(row).ravel()
        mp = np.empty(splits)
        dp = np.empty(splits)
        m, d = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_split_stats(_p(r), r.size, int(splits), _p(mp), _p(dp),
                                    ctypes.byref(m), ctypes.byref(d))
        return m.value, d.value, mp, dp

    def online_softmax(self, x, block: int) -> np.ndarray:
        x = _rows(x)
        y = np.empty_like(x)
        self.lib.oracle_online_softmax(_p(x), _p(y), x.shape[0], x.shape[1], int(block))
        return y

    def split_softmax(self, x, splits: int) -> np.ndarray:
        x = _rows(x)
        y = np.empty_like(x)
        self.lib.oracle_split_softmax(_p(x), _p(y), x.shape[0], x.shape[1], int(splits))
        return y

    def gelu_tanh(self, z) -> np.ndarray:
        z = _f64(z)
        shape = z.shape
        z = z.ravel()
        y = np.empty_like(z)
        self.lib.oracle_gelu_tanh_array(_p(z), _p(y), z.size)
        return y.reshape(shape)

    def layernorm_stats(self, row, eps: float):
        """(mean, var, rstd) of one row."""
        r = _f64(row).ravel()
        mean, var, rstd = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_layernorm_stats(_p(r), r.size, float(eps), ctypes.byref(mean),
                                        ctypes.byref(var), ctypes.byref(rstd))
        return mean.value, var.value, rstd.value

    def layernorm_normalize(self, x, eps: float) -> np.ndarray:
        x = _rows(x)
        y = np.empty_like(x)
        self.lib.oracle_layernorm_normalize(_p(x), _p(y), x.shape[0], x.shape[1], float(eps))
        return y

    def layernorm_gelu(self, x, w, b, eps: float) -> np.ndarray:
        """Fused LayerNorm + affine + tanh GeLU of a [M, N] array."""
        x = _rows(x)
        w = _f64(w).ravel()
        b = _f64(b).ravel()
        assert w.size == x.shape[1] and b.size == x.shape[1]
        y = np.empty_like(x)
        self.lib.oracle_layernorm_gelu(_p(x), _p(w), _p(b), _p(y), x.shape[0], x.shape[1],
                                       float(eps))
        return y

    def rms_stats(self, row, eps: float):
        """(mean square, inv_rms) of one row."""
        r = _f64(row).ravel()
        ms, inv = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_rms_stats(_p(r), r.size, float(eps), ctypes.byref(ms), ctypes.byref(inv))
        return ms.value, inv.value

    def rmsnorm(self, x, w, eps: float) -> np.ndarray:
        """RMSNorm of a [M, N] array: x * rsqrt(mean(x^2) + eps) * w."""
        x = _rows(x)
        w = _f64(w).ravel()
        assert w.size == x.shape[1]
        y = np.empty_like(x)
        self.lib.oracle_rmsnorm(_p(x), _p(w), _p(y), x.shape[0], x.shape[1], float(eps))
        return y

    def residual_rmsnorm(self, x, residual, w, eps: float):
        """(out, residual_out) of the fused residual RMSNorm."""
        x = _rows(x)
        res = _rows(residual)
        w = _f64(w).ravel()
        assert res.shape == x.shape and w.size == x.shape[1]
        y = np.empty_like(x)
        r = np.empty_like(x)
        self.lib.oracle_residual_rmsnorm(_p(x), _p(res), _p(w), _p(y), _p(r), x.shape[0],
                                         x.shape[1], float(eps))
        return y, r

    def gelu_erf(self, z) -> np.ndarray:
        """Exact GeLU 0.5 z (1 + erf(z / sqrt 2)), elementwise."""
        z = _f64(z)
        y = np.empty_like(z)
        self.lib.oracle_gelu_erf_array(_p(z), _p(y), z.size)
        return y

    def chunk_moments(self, row):
        """(mean, M2) of a row: M2 = sum of squared deviations from the mean."""
        r = _f64(row).ravel()
        mean, m2 = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_chunk_moments(_p(r), r.size, ctypes.byref(mean), ctypes.byref(m2))
        return mean.value, m2.value

    def chan_merge(self, a, b):
        """Combine two (n, mean, M2) summaries of disjoint parts of a row."""
        n, mean, m2 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_chan_merge(float(a[0]), float(a[1]), float(a[2]), float(b[0]),
                                   float(b[1]), float(b[2]), ctypes.byref(n), ctypes.byref(mean),
                                   ctypes.byref(m2))
        return n.value, mean.value, m2.value

    def split_moments(self, row, splits: int):
        """(mean, M2, n_parts, mean_parts, m2_parts) of the split-row statistics."""
        r = _f64(row).ravel()
        parts = [np.empty(splits) for _ in range(3)]
        mean, m2 = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_split_moments(_p(r), r.size, int(splits), _p(parts[0]), _p(parts[1]),
                                      _p(parts[2]), ctypes.byref(mean), ctypes.byref(m2))
        return (mean.value, m2.value, *parts)

    def layernorm_gelu_ex(self, x, w, b, eps: float, gelu: str = "tanh",
                          splits: int = 0) -> np.ndarray:
        """LayerNorm + affine + GeLU ("tanh" or "erf"; "none": the LayerNorm
        alone); splits = 0 takes the whole-row statistics, splits >= 1 the
        Chan-merged split statistics."""
        x = _rows(x)
        w = _f64(w).ravel()
        b = _f64(b).ravel()
        assert w.size == x.shape[1] and b.size == x.shape[1]
        kind = {"tanh": 0, "erf": 1, "none": 2}[gelu]
        y = np.empty_like(x)
        self.lib.oracle_layernorm_gelu_ex(_p(x), _p(w), _p(b), _p(y), x.shape[0], x.shape[1],
                                          float(eps), kind, int(splits))
        return y

    def row_sum(self, x) -> np.ndarray:
        """sum_j x[i, j] of a [M, N] array, in double."""
        x = _rows(x)
        out = np.empty(x.shape[0])
        self.lib.oracle_row_sum(_p(x), _p(out), x.shape[0], x.shape[1])
        return out

    def row_max(self, x) -> np.ndarray:
        """max_j x[i, j] of a [M, N] array (NaN if the row holds a NaN)."""
        x = _rows(x)
        out = np.empty(x.shape[0])
        self.lib.oracle_row_max(_p(x), _p(out), x.shape[0], x.shape[1])
        return out

    @staticmethod
    def _qkv(q, k, v):
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim < 2 or q.shape != k.shape or q.shape != v.shape:
            raise ValueError("q, k, v must share one shape [..., T, d]")
        return q, k, v

    def attention(self, q, k, v, causal: bool = False, scale: float | None = None):
        """softmax(q k^T * scale) v over the last two dimensions [..., T, d]
        (scale defaults to 1/sqrt(d)); causal: query i sees keys j <= i."""
        q, k, v = self._qkv(q, k, v)
        T, d = q.shape[-2:]
        BH = q.size // (T * d) if T * d else 0
        sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
        o = np.empty_like(q)
        self.lib.oracle_attention(_p(q), _p(k), _p(v), _p(o), BH, T, d, int(causal), sc)
        return o

    def attention_rows(self, q_rows, positions, k, v, causal: bool = False,
                       scale: float | None = None):
        """The definition for selected query rows of one (batch, head):
        q_rows [n, d] are the queries at `positions` of the sequence of k and
        v [T, d]; causal: the query at position p sees keys j <= p."""
        q, k, v = _f64(q_rows), _f64(k), _f64(v)
        pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
        if q.ndim != 2 or k.ndim != 2 or k.shape != v.shape or q.shape[1] != k.shape[1] \
                or pos.shape != (q.shape[0],):
            raise ValueError("q_rows [n, d], positions [n], k and v [T, d]")
        T, d = k.shape
        if pos.size and (pos.min() < 0 or pos.max() >= T):
            raise ValueError("positions must lie in [0, T)")
        sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
        o = np.empty_like(q)
        self.lib.oracle_attention_rows(_p(q), pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                       q.shape[0], _p(k), _p(v), _p(o), T, d, int(causal), sc)
        return o

    def flash_attention(self, q, k, v, causal: bool = False, scale: float | None = None,
                        block_q: int = 16, block_kv: int = 16):
        """The tiled online-softmax form with the given block sizes."""
        q, k, v = self._qkv(q, k, v)
        T, d = q.shape[-2:]
        BH = q.size // (T * d) if T * d else 0
        sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
        o = np.empty_like(q)
        self.lib.oracle_flash_attention(_p(q), _p(k), _p(v), _p(o), BH, T, d, int(causal), sc,
                                        int(block_q), int(block_kv))
        return o


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def _forward(name):
    def f(*args, **kw):
        return getattr(default(), name)(*args, **kw)

    f.__name__ = name
    f.__doc__ = getattr(Oracle, name).__doc__
    return f


for _n in ["softmax", "softmax_stats", "softmax_apply", "online_stats", "merge", "split_stats", "online_softmax",
           "split_softmax", "gelu_tanh", "layernorm_stats", "layernorm_normalize",
           "layernorm_gelu", "rms_stats", "rmsnorm", "residual_rmsnorm", "gelu_erf",
           "chunk_moments", "chan_merge", "split_moments", "layernorm_gelu_ex", "row_sum",
           "row_max", "attention", "flash_attention", "attention_rows"]:
    globals()[_n] = _forward(_n)
del _n
