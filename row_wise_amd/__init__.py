"""Python binding of librowkern.so (HIP kernels for MI355X / gfx950).

Argument marshalling only: every step of every operation runs in the HIP
kernels of ``librowkern.so``.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or a call fails, an
exception is raised.

Functions carry the C entry points' names:

* ``rk_softmax(x, out=None)``
* ``rk_online_softmax(x, num_splits=1, out=None, workspace=None)``
* ``rk_online_softmax_noalloc(x, num_splits=1, out=None)`` (partials in the library's fixed
  device scratch)
* ``rk_layernorm_gelu(x, weight, bias, eps=1e-5, out=None)``
* ``rk_layernorm_gelu_ex(x, weight, bias, eps=1e-5, gelu="tanh", num_splits=1, out=None,
  workspace=None)``, ``rk_layernorm_gelu_workspace_bytes(M, N, num_splits, dtype)``,
  ``rk_layernorm_gelu_auto_splits(M, N, dtype)``
* ``rk_row_sum(x, out=None)``, ``rk_row_max(x, out=None)``, ``rk_gelu(x, gelu="tanh", out=None)``
* ``rk_row_sum_ex(x, num_splits=0, out=None, workspace=None)``, ``rk_row_max_ex(...)``,
  ``rk_row_reduce_workspace_bytes(M, N, num_splits, dtype)``,
  ``rk_row_reduce_auto_splits(M, N, dtype)``
* ``rk_flash_attention(q, k, v, causal=False, scale=None, out=None)``
* ``rk_rmsnorm(x, weight, eps=1e-5, out=None)``
* ``rk_residual_rmsnorm(x, residual, weight, eps=1e-5, out=None, residual_out=None)``
* ``rk_online_softmax_workspace_bytes(M, N, num_splits, dtype)``,
  ``rk_online_softmax_auto_splits(M, N, dtype)``, ``rk_status_string(s)``,
  ``rk_version()``
* tuning: ``rk_probe_copy(src, dst)``, ``rk__softmax_variant(index, x, out)``,
  ``rk__layernorm_gelu_variant(index, x, w, b, eps, out)``, ``variants(op, dtype)``

Tensors are 2-D with unit column stride (any row stride >= N); inputs of more
than two dimensions are flattened to rows when contiguous.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LIB_PATH", "RowKernError", "load", "rk_softmax", "rk_online_softmax",
    "rk_layernorm_gelu", "rk_online_softmax_workspace_bytes", "rk_online_softmax_auto_splits",
    "rk_status_string", "rk_version", "rk_probe_copy", "rk__softmax_variant",
    "rk__layernorm_gelu_variant", "variants", "RK_F32", "RK_BF16", "RK_OP_SOFTMAX",
    "RK_OP_LAYERNORM_GELU", "rk_rmsnorm", "rk_residual_rmsnorm", "rk__rmsnorm_variant",
    "rk__residual_rmsnorm_variant", "RK_OP_RMSNORM", "RK_OP_RESIDUAL_RMSNORM",
    "rk_layernorm_gelu_ex", "rk_layernorm_gelu_workspace_bytes", "rk_layernorm_gelu_auto_splits",
    "RK_GELU_TANH", "RK_GELU_ERF", "RK_GELU_NONE", "rk_row_sum", "rk_row_max", "rk_gelu", "rk_flash_attention",
    "RK_F16", "rk_online_softmax_noalloc", "rk_row_sum_ex", "rk_row_max_ex",
    "rk_row_reduce_workspace_bytes", "rk_row_reduce_auto_splits",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librowkern.so")

RK_F32, RK_BF16, RK_F16 = 0, 1, 2
RK_OP_SOFTMAX, RK_OP_LAYERNORM_GELU, RK_OP_RMSNORM, RK_OP_RESIDUAL_RMSNORM = 0, 1, 2, 3
RK_GELU_TANH, RK_GELU_ERF, RK_GELU_NONE = 0, 1, 2
_GELU = {"tanh": RK_GELU_TANH, "erf": RK_GELU_ERF, "none": RK_GELU_NONE}
RK_OK = 0


class RowKernError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {rk_status_string(status)} (status {status})")


_lib = None


def load():
    """Load librowkern.so (raising if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m row_wise_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz, f32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                             ctypes.c_float)
    sig = {
        "rk_softmax": (i32, [vp, vp, i64, i64, i64, i64, i32, vp]),
        "rk_online_softmax": (i32, [vp, vp, i64, i64, i64, i64, i32, i32, vp, sz, vp]),
        "rk_online_softmax_noalloc": (i32, [vp, vp, i64, i64, i64, i64, i32, i32, vp]),
        "rk_online_softmax_workspace_bytes": (sz, [i64, i64, i32, i32]),
        "rk_online_softmax_auto_splits": (i32, [i64, i64, i32]),
        "rk_layernorm_gelu": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, vp]),
        "rk_status_string": (ctypes.c_char_p, [i32]),
        "rk_version": (ctypes.c_int, []),
        "rk_probe_copy": (i32, [vp, vp, sz, i32, vp]),
        "rk__variant_count": (i32, [i32, i32]),
        "rk__variant_info": (i32, [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                   ctypes.POINTER(i32), ctypes.POINTER(i32),
                                   ctypes.POINTER(i64), ctypes.POINTER(i32),
                                   ctypes.POINTER(i32)]),
        "rk__variant_pick": (i32, [i32, i32, i64]),
        "rk__softmax_variant": (i32, [i32, vp, vp, i64, i64, i64, i64, i32, vp]),
        "rk__layernorm_gelu_variant": (i32, [i32, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32,
                                             i32, vp]),
        "rk_layernorm_gelu_ex": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, i32, vp,
                                       sz, vp]),
        "rk_layernorm_gelu_workspace_bytes": (sz, [i64, i64, i32, i32]),
        "rk_layernorm_gelu_auto_splits": (i32, [i64, i64, i32]),
        "rk_row_sum": (i32, [vp, vp, i64, i64, i64, i32, vp]),
        "rk_flash_attention": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, f32, i32,
                                     i32, vp]),
        "rk_row_max": (i32, [vp, vp, i64, i64, i64, i32, vp]),
        "rk_row_sum_ex": (i32, [vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]),
        "rk_row_max_ex": (i32, [vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]),
        "rk_row_reduce_workspace_bytes": (sz, [i64, i64, i32, i32]),
        "rk_row_reduce_auto_splits": (i32, [i64, i64, i32]),
        "rk_gelu": (i32, [vp, vp, i64, i64, i64, i64, i32, i32, vp]),
        "rk_rmsnorm": (i32, [vp, vp, vp, i64, i64, i64, i64, f32, i32, vp]),
        "rk_residual_rmsnorm": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32,
                                      vp]),
        "rk__rmsnorm_variant": (i32, [i32, vp, vp, vp, i64, i64, i64, i64, f32, i32, vp]),
        "rk__residual_rmsnorm_variant": (i32, [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                               i64, f32, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---------------------------------------------------------------- helpers


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RK_F32
    if t.dtype == torch.bfloat16:
        return RK_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _as_rows(x):
    """View x as [M, N] rows with unit column stride; returns (view, M, N, ld)."""
    if x.dim() == 1:
        v = x.reshape(1, -1)
    elif x.dim() == 2:
        v = x
    elif x.is_contiguous():
        v = x.reshape(-1, x.shape[-1])
    else:
        raise ValueError("inputs of more than two dimensions must be contiguous")
    M, N = v.shape
    if M > 0 and N > 1 and v.stride(1) != 1:
        raise ValueError("rows must have unit column stride")
    ld = v.stride(0) if M > 1 else N
    if M > 1 and ld < N:
        raise ValueError("rows overlap (row stride < N)")
    return v, M, N, ld


def _stream(t) -> int:
    torch = _torch()
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return 0


def _check_device(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _call(name: str, *args) -> None:
    st = getattr(load(), name)(*args)
    if st != RK_OK:
        raise RowKernError(name, st)


def _out_like(x, v, out):
    """Output rows for input rows v: a new tensor, or `out` checked; (rows, ld)."""
    torch = _torch()
    if out is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    else:
        if out.dtype != x.dtype or out.device != x.device:
            raise ValueError("out must have the input's dtype and device")
        o = out
    o, Mo, No, ldo = _as_rows(o)
    if (Mo, No) != tuple(v.shape):
        raise ValueError("out must have the input's rows and columns")
    return o, ldo


# ------------------------------------------------------------- entry points


def rk_status_string(status: int) -> str:
    return load().rk_status_string(int(status)).decode()


def rk_version() -> int:
    return int(load().rk_version())


def rk_online_softmax_workspace_bytes(M: int, N: int, num_splits: int, dtype: int) -> int:
    return int(load().rk_online_softmax_workspace_bytes(M, N, num_splits, dtype))


def rk_online_softmax_auto_splits(M: int, N: int, dtype: int) -> int:
    return int(load().rk_online_softmax_auto_splits(M, N, dtype))


def rk_softmax(x, out=None):
    """Stable row softmax of x (rows = last dimension); returns y."""
    _check_device(x)
    v, M, N, ldx = _as_rows(x)
    o, ldy = _out_like(x, v, out)
    _call("rk_softmax", v.data_ptr(), o.data_ptr(), M, N, ldx, ldy, _dtype_code(x), _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk_online_softmax(x, num_splits: int = 1, out=None, workspace=None):
    """Online softmax (num_splits 1: streaming; >= 2: split-row; 0: auto)."""
    torch = _torch()
    _check_device(x)
    v, M, N, ldx = _as_rows(x)
    o, ldy = _out_like(x, v, out)
    need = rk_online_softmax_workspace_bytes(M, N, num_splits, _dtype_code(x)) if M > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("rk_online_softmax", v.data_ptr(), o.data_ptr(), M, N, ldx, ldy, _dtype_code(x),
          int(num_splits), wptr, wbytes, _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk_online_softmax_noalloc(x, num_splits: int = 1, out=None):
    """rk_online_softmax with the split partials in the library's fixed device
    scratch instead of a workspace (the library allocates nothing)."""
    _check_device(x)
    v, M, N, ldx = _as_rows(x)
    o, ldy = _out_like(x, v, out)
    _call("rk_online_softmax_noalloc", v.data_ptr(), o.data_ptr(), M, N, ldx, ldy,
          _dtype_code(x), int(num_splits), _stream(x))
    return o.reshape(x.shape) if out is None else out


def _check_affine(weight, bias, x, N):
    if weight.shape != (N,) or bias.shape != (N,) or not weight.is_contiguous() \
            or not bias.is_contiguous():
        raise ValueError("weight and bias must be contiguous [N]")
    if weight.dtype != x.dtype or bias.dtype != x.dtype:
        raise ValueError("weight and bias must have the input's dtype")


def rk_layernorm_gelu(x, weight, bias, eps: float = 1e-5, out=None):
    """Fused LayerNorm + affine + tanh GeLU over the last dimension."""
    _check_device(x, weight, bias)
    v, M, N, ldx = _as_rows(x)
    _check_affine(weight, bias, x, N)
    o, ldy = _out_like(x, v, out)
    _call("rk_layernorm_gelu", v.data_ptr(), weight.data_ptr(), bias.data_ptr(), o.data_ptr(),
          M, N, ldx, ldy, float(eps), _dtype_code(x), _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk_layernorm_gelu_workspace_bytes(M: int, N: int, num_splits: int, dtype: int) -> int:
    return int(load().rk_layernorm_gelu_workspace_bytes(M, N, num_splits, dtype))


def rk_layernorm_gelu_auto_splits(M: int, N: int, dtype: int) -> int:
    return int(load().rk_layernorm_gelu_auto_splits(M, N, dtype))


def rk_layernorm_gelu_ex(x, weight, bias, eps: float = 1e-5, gelu: str = "tanh",
                         num_splits: int = 1, out=None, workspace=None):
    """LayerNorm + affine + GeLU ("tanh" or "erf"; "none": the LayerNorm
    alone); num_splits 1: one workgroup or tile per row, >= 2: split-row, 0:
    auto."""
    torch = _torch()
    _check_device(x, weight, bias)
    v, M, N, ldx = _as_rows(x)
    _check_affine(weight, bias, x, N)
    o, ldy = _out_like(x, v, out)
    dt = _dtype_code(x)
    need = rk_layernorm_gelu_workspace_bytes(M, N, num_splits, dt) if M > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("rk_layernorm_gelu_ex", v.data_ptr(), weight.data_ptr(), bias.data_ptr(), o.data_ptr(),
          M, N, ldx, ldy, float(eps), dt, _GELU[gelu], int(num_splits), wptr, wbytes, _stream(x))
    return o.reshape(x.shape) if out is None else out


def _row_reduce(name, x, out):
    torch = _torch()
    _check_device(x)
    v, M, N, ldx = _as_rows(x)
    shape = x.shape[:-1] if x.dim() > 1 else ()
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif out.shape != shape or out.dtype != x.dtype or out.device != x.device \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of the input's rows, dtype and device")
    _call(name, v.data_ptr(), out.data_ptr(), M, N, ldx, _dtype_code(x), _stream(x))
    return out


def rk_row_sum(x, out=None):
    """sum over the last dimension (fp32 accumulation, result in x's dtype)."""
    return _row_reduce("rk_row_sum", x, out)


def rk_row_max(x, out=None):
    """max over the last dimension (NaN if a row holds a NaN)."""
    return _row_reduce("rk_row_max", x, out)


def rk_row_reduce_workspace_bytes(M: int, N: int, num_splits: int, dtype: int) -> int:
    return int(load().rk_row_reduce_workspace_bytes(M, N, num_splits, dtype))


def rk_row_reduce_auto_splits(M: int, N: int, dtype: int) -> int:
    return int(load().rk_row_reduce_auto_splits(M, N, dtype))


def _row_reduce_ex(name, x, num_splits, out, workspace):
    torch = _torch()
    _check_device(x)
    v, M, N, ldx = _as_rows(x)
    shape = x.shape[:-1] if x.dim() > 1 else ()
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif out.shape != shape or out.dtype != x.dtype or out.device != x.device \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of the input's rows, dtype and device")
    dt = _dtype_code(x)
    need = rk_row_reduce_workspace_bytes(M, N, num_splits, dt) if M > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call(name, v.data_ptr(), out.data_ptr(), M, N, ldx, dt, int(num_splits), wptr, wbytes,
          _stream(x))
    return out


def rk_row_sum_ex(x, num_splits: int = 0, out=None, workspace=None):
    """rk_row_sum with long rows split across workgroups (num_splits 0: auto,
    1: one workgroup per row, >= 2: that many chunks per row)."""
    return _row_reduce_ex("rk_row_sum_ex", x, num_splits, out, workspace)


def rk_row_max_ex(x, num_splits: int = 0, out=None, workspace=None):
    """rk_row_max with long rows split across workgroups (as rk_row_sum_ex)."""
    return _row_reduce_ex("rk_row_max_ex", x, num_splits, out, workspace)


def rk_gelu(x, gelu: str = "tanh", out=None):
    """Elementwise GeLU ("tanh" approximation or exact "erf")."""
    _check_device(x)
    v, M, N, ldx = _as_rows(x)
    o, ldy = _out_like(x, v, out)
    _call("rk_gelu", v.data_ptr(), o.data_ptr(), M, N, ldx, ldy, _dtype_code(x), _GELU[gelu],
          _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk_flash_attention(q, k, v, causal: bool = False, scale=None, out=None):
    """softmax(q k^T * scale) v for [B, H, T, d] tensors (bf16 or fp16, unit
    stride along d); scale defaults to 1 / sqrt(d)."""
    torch = _torch()
    _check_device(q, k, v)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, T, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    B, H, T, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError("out must match q")
    for t in (q, k, v, out):
        if T > 0 and d > 1 and t.stride(3) != 1:
            raise ValueError("the head dimension must have unit stride")
    code = {torch.bfloat16: RK_BF16, torch.float16: RK_F16, torch.float32: RK_F32}.get(q.dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    sc = 1.0 / (d ** 0.5) if scale is None else float(scale)

    def strides(t):
        return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))

    arrs = [strides(t) for t in (q, k, v, out)]  # alive for the call
    sq, sk, sv, so = (ctypes.cast(a, ctypes.c_void_p) for a in arrs)
    _call("rk_flash_attention", q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H,
          T, d, sq, sk, sv, so, sc, int(bool(causal)), code, _stream(q))
    return out


def _check_weight(weight, x, N):
    if weight.shape != (N,) or not weight.is_contiguous():
        raise ValueError("weight must be contiguous [N]")
    if weight.dtype != x.dtype:
        raise ValueError("weight must have the input's dtype")


def rk_rmsnorm(x, weight, eps: float = 1e-5, out=None):
    """RMSNorm over the last dimension: x * rsqrt(mean(x^2) + eps) * weight."""
    _check_device(x, weight)
    v, M, N, ldx = _as_rows(x)
    _check_weight(weight, x, N)
    o, ldy = _out_like(x, v, out)
    _call("rk_rmsnorm", v.data_ptr(), weight.data_ptr(), o.data_ptr(), M, N, ldx, ldy,
          float(eps), _dtype_code(x), _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk_residual_rmsnorm(x, residual, weight, eps: float = 1e-5, out=None, residual_out=None):
    """(y, residual_out): residual_out = x + residual, y = RMSNorm(residual_out)."""
    _check_device(x, residual, weight)
    v, M, N, ldx = _as_rows(x)
    if residual.shape != x.shape or residual.dtype != x.dtype:
        raise ValueError("residual must match x")
    rv, _, _, ldr = _as_rows(residual)
    _check_weight(weight, x, N)
    o, ldy = _out_like(x, v, out)
    ro, ldo = _out_like(x, v, residual_out)
    _call("rk_residual_rmsnorm", v.data_ptr(), rv.data_ptr(), weight.data_ptr(), o.data_ptr(),
          ro.data_ptr(), M, N, ldx, ldr, ldy, ldo, float(eps), _dtype_code(x), _stream(x))
    y = o.reshape(x.shape) if out is None else out
    r = ro.reshape(x.shape) if residual_out is None else residual_out
    return y, r


# ------------------------------------------------------------------ tuning


def rk_probe_copy(src, dst, max_workgroups: int = 0):
    """16-byte copy kernel over the bytes of src into dst (same size)."""
    _check_device(src, dst)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _call("rk_probe_copy", src.data_ptr(), dst.data_ptr(), nbytes, int(max_workgroups),
          _stream(src))


def variants(op: int, dtype: int) -> list[dict]:
    """Geometry of every compiled tile variant of op (RK_OP_*) for dtype."""
    lib = load()
    out = []
    for i in range(lib.rk__variant_count(op, dtype)):
        g, v, w, r, ex, alt = (ctypes.c_int32() for _ in range(6))
        n = ctypes.c_int64()
        st = lib.rk__variant_info(op, dtype, i, ctypes.byref(g), ctypes.byref(v), ctypes.byref(w),
                                  ctypes.byref(r), ctypes.byref(n), ctypes.byref(ex),
                                  ctypes.byref(alt))
        if st != RK_OK:
            raise RowKernError("rk__variant_info", st)
        out.append({"index": i, "waves_per_row": g.value, "vecs_per_lane": v.value,
                    "waves_per_block": w.value, "rows_per_group": r.value, "max_n": n.value,
                    "exact": bool(ex.value), "alternative": bool(alt.value)})
    return out


def variant_pick(op: int, dtype: int, N: int) -> int:
    return int(load().rk__variant_pick(op, dtype, N))


def rk__softmax_variant(index: int, x, out=None):
    _check_device(x)
    v, M, N, ldx = _as_rows(x)
    o, ldy = _out_like(x, v, out)
    _call("rk__softmax_variant", int(index), v.data_ptr(), o.data_ptr(), M, N, ldx, ldy,
          _dtype_code(x), _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk__layernorm_gelu_variant(index: int, x, weight, bias, eps: float = 1e-5, out=None,
                               gelu: str = "tanh"):
    _check_device(x, weight, bias)
    v, M, N, ldx = _as_rows(x)
    o, ldy = _out_like(x, v, out)
    _call("rk__layernorm_gelu_variant", int(index), v.data_ptr(), weight.data_ptr(),
          bias.data_ptr(), o.data_ptr(), M, N, ldx, ldy, float(eps), _dtype_code(x), _GELU[gelu],
          _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk__rmsnorm_variant(index: int, x, weight, eps: float = 1e-5, out=None):
    _check_device(x, weight)
    v, M, N, ldx = _as_rows(x)
    o, ldy = _out_like(x, v, out)
    _call("rk__rmsnorm_variant", int(index), v.data_ptr(), weight.data_ptr(), o.data_ptr(), M, N,
          ldx, ldy, float(eps), _dtype_code(x), _stream(x))
    return o.reshape(x.shape) if out is None else out


def rk__residual_rmsnorm_variant(index: int, x, residual, weight, eps: float = 1e-5, out=None,
                                 residual_out=None):
    _check_device(x, residual, weight)
    v, M, N, ldx = _as_rows(x)
    rv, _, _, ldr = _as_rows(residual)
    o, ldy = _out_like(x, v, out)
    ro, ldo = _out_like(x, v, residual_out)
    _call("rk__residual_rmsnorm_variant", int(index), v.data_ptr(), rv.data_ptr(),
          weight.data_ptr(), o.data_ptr(), ro.data_ptr(), M, N, ldx, ldr, ldy, ldo, float(eps),
          _dtype_code(x), _stream(x))
    y = o.reshape(x.shape) if out is None else out
    r = ro.reshape(x.shape) if residual_out is None else residual_out
    return y, r
