"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects invalid arguments before any HIP call.  (Nothing here
launches a kernel.)"""
import ctypes
import glob
import os
import re

import pytest

import row_wise_amd as rk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
F32, BF16 = rk.RK_F32, rk.RK_BF16
A = 0x100000  # fake, 16-byte aligned device addresses: never dereferenced
B = 0x900000
INT32_MAX = 2**31 - 1


@pytest.fixture(scope="module")
def lib():
    return rk.load()


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(rk_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert {"rk_softmax", "rk_online_softmax", "rk_layernorm_gelu"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_only_rk_symbols_exported():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", rk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    text_syms = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert text_syms and all(s.startswith("rk_") for s in text_syms), text_syms
    assert set(text_syms) == set(declared_symbols())


def test_status_strings_and_version(lib):
    assert rk.rk_version() == 100
    assert rk.rk_status_string(0) == "ok"
    assert rk.rk_status_string(INVALID) == "invalid argument"
    assert rk.rk_status_string(WORKSPACE) == "workspace missing or too small"
    assert rk.rk_status_string(99) == "unknown status"


def sm(lib, x=A, y=B, M=4, N=8, ldx=None, ldy=None, dt=F32):
    return lib.rk_softmax(x, y, M, N, N if ldx is None else ldx, N if ldy is None else ldy, dt,
                          None)


@pytest.mark.parametrize("kw", [
    dict(dt=2), dict(dt=-1), dict(M=-1), dict(N=0), dict(N=-3), dict(N=INT32_MAX + 1,
                                                                    ldx=2**32, ldy=2**32),
    dict(ldx=7), dict(ldy=7), dict(x=None), dict(y=None), dict(x=A + 2), dict(y=B + 1, dt=BF16),
    dict(y=A + 16), dict(x=A, y=A, ldx=8, ldy=16), dict(M=2**62, ldx=2**20, ldy=2**20),
])
def test_softmax_rejects(lib, kw):
    assert sm(lib, **kw) == INVALID


def test_rows_beyond_2_30_unsupported(lib):
    n = 2**30 + 1
    assert sm(lib, M=1, N=n) == UNSUPPORTED


def test_tallest_grid_refused_before_launch(lib):
    # 2^26 rows of 8 on a one-wave-per-row tile need 2^32 work-items: refused
    # before any HIP call (2^26 - 4 rows, the largest accepted, run on the GPU)
    X = 0x10000000
    assert lib.rk_softmax(X, X, 1 << 26, 8, 8, 8, F32, None) == UNSUPPORTED
    assert lib.rk_layernorm_gelu(X, 0x100000, 0x200000, X, 1 << 26, 8, 8, 8, 1e-5, F32,
                                 None) == UNSUPPORTED


def test_m_zero_is_a_noop(lib):
    assert sm(lib, x=None, y=None, M=0) == 0
    assert lib.rk_online_softmax(None, None, 0, 8, 8, 8, F32, 64, None, 0, None) == 0
    assert lib.rk_layernorm_gelu(None, None, None, None, 0, 8, 8, 8, 1e-5, F32, None) == 0
    assert lib.rk_rmsnorm(None, None, None, 0, 8, 8, 8, 1e-5, F32, None) == 0
    assert lib.rk_residual_rmsnorm(None, None, None, None, None, 0, 8, 8, 8, 8, 8, 1e-5, F32,
                                   None) == 0
    # but sizes are still checked
    assert sm(lib, x=None, y=None, M=0, N=0) == INVALID


def ln(lib, x=A, w=A + 0x80000, b=A + 0x90000, y=B, M=4, N=8, ldx=8, ldy=8, eps=1e-5, dt=F32):
    return lib.rk_layernorm_gelu(x, w, b, y, M, N, ldx, ldy, eps, dt, None)


@pytest.mark.parametrize("kw", [
    dict(eps=0.0), dict(eps=-1e-5), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(w=None), dict(b=None), dict(x=None), dict(w=B + 8), dict(b=B), dict(dt=7), dict(N=0),
    dict(ldy=4), dict(w=A + 0x80001), dict(y=A + 64),
])
def test_layernorm_rejects(lib, kw):
    assert ln(lib, **kw) == INVALID


def rms(lib, x=A, w=A + 0x80000, y=B, M=4, N=8, ldx=8, ldy=8, eps=1e-5, dt=F32):
    return lib.rk_rmsnorm(x, w, y, M, N, ldx, ldy, eps, dt, None)


@pytest.mark.parametrize("kw", [
    dict(eps=0.0), dict(eps=-1.0), dict(eps=float("nan")), dict(eps=float("inf")), dict(w=None),
    dict(x=None), dict(y=None), dict(w=B + 8), dict(w=A + 0x80002), dict(dt=3), dict(N=0),
    dict(ldx=7), dict(y=A + 32), dict(x=A + 1, dt=BF16),
])
def test_rmsnorm_rejects(lib, kw):
    assert rms(lib, **kw) == INVALID


C = 0x1100000
D = 0x1900000


def res_rms(lib, x=A, r=C, w=A + 0x80000, y=B, ro=D, M=4, N=8, ldx=8, ldr=8, ldy=8, ldo=8,
            eps=1e-5, dt=F32):
    return lib.rk_residual_rmsnorm(x, r, w, y, ro, M, N, ldx, ldr, ldy, ldo, eps, dt, None)


@pytest.mark.parametrize("kw", [
    dict(eps=0.0), dict(eps=float("nan")), dict(w=None), dict(r=None), dict(ro=None),
    dict(x=None), dict(y=None), dict(dt=2), dict(N=0), dict(M=-1), dict(ldr=7), dict(ldo=7),
    dict(ro=D + 2), dict(r=C + 2, dt=F32),
    dict(ro=B),  # the two outputs coincide
    dict(ro=B + 64),  # the outputs overlap
    dict(ro=A + 0x80000 - 16),  # residual_out overlaps the weight
    dict(y=A + 0x80000),  # y is the weight
    dict(ro=A + 16),  # partial overlap with x
    dict(y=C + 32),  # partial overlap with residual
    dict(ro=C, ldo=16),  # same pointer, other pitch
])
def test_residual_rmsnorm_rejects(lib, kw):
    assert res_rms(lib, **kw) == INVALID


def test_residual_rmsnorm_limits(lib):
    n = 2**30 + 1
    assert res_rms(lib, M=1, N=n, ldx=n, ldr=n, ldy=n, ldo=n) == UNSUPPORTED
    assert rms(lib, M=1, N=n, ldx=n, ldy=n) == UNSUPPORTED


def lnx(lib, x=A, w=A + 0x80000, b=A + 0x90000, y=B, M=4, N=4096, ldx=4096, ldy=4096, eps=1e-5,
        dt=F32, gelu=0, S=8, ws=0x3000000, wb=4 * 9 * 8):
    return lib.rk_layernorm_gelu_ex(x, w, b, y, M, N, ldx, ldy, eps, dt, gelu, S, ws, wb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(gelu=3), INVALID), (dict(gelu=-1), INVALID), (dict(S=-1), INVALID),
    (dict(S=65537), INVALID), (dict(eps=0.0), INVALID), (dict(b=None), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wb=4 * 9 * 8 - 1), WORKSPACE),
    (dict(ws=0x3000004), INVALID),  # misaligned workspace
    (dict(ws=A + 64), INVALID),  # workspace overlaps x
    (dict(ws=A + 0x80000 - 8), INVALID),  # workspace overlaps the weight
    (dict(ws=B + 4096 * 4 * 3), INVALID),  # workspace overlaps y
    (dict(N=2**30 + 1, ldx=2**30 + 1, ldy=2**30 + 1), UNSUPPORTED),
])
def test_layernorm_ex_rejects(lib, kw, status):
    assert lnx(lib, **kw) == status


def test_layernorm_ex_workspace_and_splits(lib):
    assert rk.rk_layernorm_gelu_workspace_bytes(64, 262144, 64, F32) == 64 * 65 * 8
    assert rk.rk_layernorm_gelu_workspace_bytes(64, 262144, 1, F32) == 0
    assert rk.rk_layernorm_gelu_workspace_bytes(64, 262144, -1, F32) == 0
    assert rk.rk_layernorm_gelu_workspace_bytes(64, 262144, 4, 9) == 0
    # rows a register tile holds are not split by default
    assert rk.rk_layernorm_gelu_auto_splits(8, 16384, F32) == 1
    assert rk.rk_layernorm_gelu_auto_splits(8, 32768, BF16) == 1
    assert rk.rk_layernorm_gelu_auto_splits(8, 16385, F32) > 1
    assert rk.rk_layernorm_gelu_auto_splits(4096, 65536, F32) == 1
    s = rk.rk_layernorm_gelu_auto_splits(64, 262144, F32)
    assert s >= 2 and rk.rk_layernorm_gelu_workspace_bytes(64, 262144, 0, F32) == 64 * (s + 1) * 8
    # S = 1 needs no workspace and M = 0 is a no-op
    assert lnx(lib, M=0, x=None, y=None, ws=None) == 0
    assert lib.rk_layernorm_gelu_ex(None, None, None, None, 0, 8, 8, 8, 1e-5, F32, 1, 1, None, 0,
                                    None) == 0


@pytest.mark.parametrize("fn", ["rk_row_sum", "rk_row_max"])
def test_row_reduce_rejects(lib, fn):
    f = getattr(lib, fn)
    assert f(None, B, 4, 8, 8, F32, None) == INVALID
    assert f(A, None, 4, 8, 8, F32, None) == INVALID
    assert f(A, B, -1, 8, 8, F32, None) == INVALID
    assert f(A, B, 4, 0, 8, F32, None) == INVALID
    assert f(A, B, 4, 8, 7, F32, None) == INVALID
    assert f(A, B, 4, 8, 8, 5, None) == INVALID
    assert f(A + 2, B, 4, 8, 8, F32, None) == INVALID
    assert f(A, B + 1, 4, 8, 8, BF16, None) == INVALID
    assert f(A, A + 64, 4, 8, 8, F32, None) == INVALID  # out inside x
    assert f(A, A - 8, 4, 8, 8, F32, None) == INVALID  # out overlaps x's start
    assert f(None, None, 0, 8, 8, F32, None) == 0
    assert f(A, B, 1, 2**30 + 1, 2**30 + 1, F32, None) == UNSUPPORTED


def rsx(lib, fn="rk_row_sum_ex", x=A, out=B, M=4, N=4096, ldx=4096, dt=F32, S=8,
        ws=0x3000000, wb=4 * 8 * 4):
    return getattr(lib, fn)(x, out, M, N, ldx, dt, S, ws, wb, None)


@pytest.mark.parametrize("fn", ["rk_row_sum_ex", "rk_row_max_ex"])
@pytest.mark.parametrize("kw,status", [
    (dict(S=-1), INVALID), (dict(S=65537), INVALID), (dict(N=0), INVALID),
    (dict(ldx=4095), INVALID), (dict(dt=5), INVALID), (dict(x=None), INVALID),
    (dict(out=A + 64), INVALID),  # out inside x
    (dict(ws=None), WORKSPACE), (dict(wb=4 * 8 * 4 - 1), WORKSPACE),
    (dict(ws=0x3000004), INVALID),  # misaligned workspace
    (dict(ws=A + 64), INVALID),  # workspace overlaps x
    (dict(ws=B - 8), INVALID),  # workspace overlaps out
    (dict(N=2**30 + 1, ldx=2**30 + 1), UNSUPPORTED),
])
def test_row_reduce_ex_rejects(lib, fn, kw, status):
    assert rsx(lib, fn, **kw) == status


def test_row_reduce_ex_workspace_and_splits(lib):
    assert rk.rk_row_reduce_workspace_bytes(64, 262144, 32, F32) == 64 * 32 * 4
    assert rk.rk_row_reduce_workspace_bytes(64, 262144, 1, F32) == 0
    assert rk.rk_row_reduce_workspace_bytes(64, 262144, -1, F32) == 0
    assert rk.rk_row_reduce_workspace_bytes(64, 262144, 4, 9) == 0
    assert rk.rk_row_reduce_workspace_bytes(0, 10, 4, F32) == 0
    for dt, es in ((F32, 4), (BF16, 2)):
        for M, N in ((1, 1 << 20), (4, 262144), (64, 262144), (16, 262144)):
            s = rk.rk_row_reduce_auto_splits(M, N, dt)
            assert s == min(-(-N * es // 16384), 2048 // M), (M, N)
            assert rk.rk_row_reduce_workspace_bytes(M, N, 0, dt) == M * s * 4
        # a full chip of rows, or rows one workgroup reads about as fast as
        # the split's two launches take
        for M, N in ((256, 1 << 20), (8192, 1000), (16384, 4096), (200, 65536), (128, 65536)):
            assert rk.rk_row_reduce_auto_splits(M, N, dt) == 1, (M, N)
    # S = 1 needs no workspace; M = 0 is a no-op
    assert rsx(lib, M=0, x=None, out=None, ws=None) == 0
    assert lib.rk_row_sum_ex(None, None, 0, 8, 8, F32, 1, None, 0, None) == 0


def test_gelu_rejects(lib):
    g = lib.rk_gelu
    assert g(A, B, 4, 8, 8, 8, F32, 2, None) == INVALID  # RK_GELU_NONE: LayerNorm only
    assert g(A, B, 4, 8, 8, 8, F32, -1, None) == INVALID
    assert g(A, A + 16, 4, 8, 8, 8, F32, 0, None) == INVALID
    assert g(None, B, 4, 8, 8, 8, F32, 0, None) == INVALID
    assert g(A, B, 4, 8, 8, 7, F32, 1, None) == INVALID
    assert g(None, None, 0, 8, 8, 8, F32, 0, None) == 0


def attn(lib, q=A, k=B, v=0x2000000, o=0x3000000, Bn=2, H=3, T=100, d=128, st=None, scale=0.1,
         causal=0, dt=BF16):
    arr = None
    if st is not None:
        arr = (ctypes.c_int64 * 3)(*st)
    sp = ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None
    return lib.rk_flash_attention(q, k, v, o, Bn, H, T, d, None, None, None, sp, scale, causal,
                                  dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), INVALID), (dict(Bn=-1), INVALID), (dict(d=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-0.5), INVALID),
    (dict(causal=2), INVALID), (dict(q=None), INVALID), (dict(o=None), INVALID),
    (dict(o=A + 4096), INVALID),  # o overlaps q
    (dict(o=0x2000000 - 64), INVALID),  # o overlaps v
    (dict(st=(3 * 100 * 128, 100 * 128, 64)), INVALID),  # seq stride < d
    (dict(st=(3 * 100 * 128, 0, 128)), INVALID),  # heads of o on top of each other
    (dict(st=(0, 100 * 128, 128)), INVALID),  # batches of o on top of each other
    (dict(dt=F32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(q=A + 2), UNSUPPORTED), (dict(st=(3 * 100 * 136, 100 * 136, 132)), UNSUPPORTED),
    (dict(Bn=0), 0), (dict(T=0, q=None, k=None, v=None, o=None), 0),
])
def test_attention_rejects(lib, kw, status):
    assert attn(lib, **kw) == status


def test_attention_layouts_accepted_by_validation(lib):
    # a [B, T, H, d] output layout nests (no overlap): only alignment or launch
    # can stop it, and M = 0 style no-ops need no pointers
    assert lib.rk_flash_attention(None, None, None, None, 2, 0, 100, 128, None, None, None,
                                  None, 0.1, 1, BF16, None) == 0


def online(lib, x=A, y=B, M=4, N=4096, S=64, ws=A + 0x400000, wb=4 * 64 * 8, dt=F32):
    return lib.rk_online_softmax(x, y, M, N, N, N, dt, S, ws, wb, None)


def test_online_rejects(lib):
    assert online(lib, S=-1) == INVALID
    assert online(lib, S=65537) == INVALID
    assert online(lib, ws=None) == WORKSPACE
    assert online(lib, wb=4 * 64 * 8 - 1) == WORKSPACE
    assert online(lib, ws=A + 0x400004) == INVALID  # misaligned workspace
    assert online(lib, ws=A + 16) == INVALID  # workspace overlaps x
    assert online(lib, N=0) == INVALID


def test_online_noalloc_rejects(lib):
    X, Y = 0x10000000, 0x20000000

    def f(M=4, N=4096, S=64, x=X, y=Y, dt=F32):
        return lib.rk_online_softmax_noalloc(x, y, M, N, N, N, dt, S, None)

    assert f(S=-1) == INVALID and f(S=65537) == INVALID and f(N=0) == INVALID
    assert f(y=X + 64) == INVALID  # y overlaps x
    assert f(M=0, x=None, y=None) == 0
    # partials beyond the 1 MiB scratch (131072 pairs): refused before any
    # HIP call
    assert f(M=2049, S=64) == 5 and f(M=3, N=2**20, S=65536) == 5
    assert rk.rk_status_string(5).startswith("split partials exceed")


def test_workspace_bytes(lib):
    assert rk.rk_online_softmax_workspace_bytes(64, 262144, 64, F32) == 64 * 64 * 8
    assert rk.rk_online_softmax_workspace_bytes(64, 262144, 1, F32) == 0
    assert rk.rk_online_softmax_workspace_bytes(64, 262144, -1, F32) == 0
    assert rk.rk_online_softmax_workspace_bytes(0, 10, 4, F32) == 0
    assert rk.rk_online_softmax_workspace_bytes(64, 262144, 4, 9) == 0
    for dt in (F32, BF16):
        s = rk.rk_online_softmax_auto_splits(64, 262144, dt)
        assert s >= 2 and rk.rk_online_softmax_workspace_bytes(64, 262144, 0, dt) == 64 * s * 8
    assert rk.rk_online_softmax_auto_splits(16384, 4096, F32) == 1
    assert rk.rk_online_softmax_auto_splits(1, 10, F32) == 1
    assert rk.rk_online_softmax_auto_splits(64, 262144, 9) == 1


@pytest.mark.parametrize("dt", [F32, BF16])
def test_auto_split_policy(dt):
    """Splits only where rows are long and too few to fill the chip, with
    chunks of about 16 KiB and at most 2048 workgroups."""
    es = 4 if dt == F32 else 2
    for M, N in ((1, 1 << 20), (4, 262144), (16, 65536), (64, 262144), (32, 131072),
                 (128, 131072), (128, 65536)):
        s = rk.rk_online_softmax_auto_splits(M, N, dt)
        assert 2 <= s and M * s <= 2048, (M, N)
        assert s == min(-(-N * es // 16384), 2048 // M), (M, N)
    # a full chip of rows, or rows one CU streams quickly: one kernel
    for M, N in ((256, 1 << 20), (4096, 65536), (200, 65536), (200, 16384), (128, 16384),
                 (1, 2048)):
        assert rk.rk_online_softmax_auto_splits(M, N, dt) == 1, (M, N)
    # LayerNorm+GeLU: rows past the register tiles follow the same rule
    assert rk.rk_layernorm_gelu_auto_splits(64, 262144, dt) == \
        rk.rk_online_softmax_auto_splits(64, 262144, dt)
    assert rk.rk_layernorm_gelu_auto_splits(256, 262144, dt) == 1


def test_probe_copy_rejects(lib):
    assert lib.rk_probe_copy(A, B, 0, 0, None) == 0
    assert lib.rk_probe_copy(A + 4, B, 64, 0, None) == INVALID
    assert lib.rk_probe_copy(A, B, 60, 0, None) == INVALID
    assert lib.rk_probe_copy(A, A + 32, 64, 0, None) == INVALID
    assert lib.rk_probe_copy(None, B, 64, 0, None) == INVALID


OPS = (rk.RK_OP_SOFTMAX, rk.RK_OP_LAYERNORM_GELU, rk.RK_OP_RMSNORM, rk.RK_OP_RESIDUAL_RMSNORM)


def test_variant_tables():
    for op in OPS:
        for dt, E, cap in ((F32, 4, 16384), (BF16, 8, 32768)):
            vs = rk.variants(op, dt)
            assert vs
            for v in vs:
                assert v["max_n"] == v["waves_per_row"] * v["vecs_per_lane"] * 64 * E
                assert v["waves_per_block"] % v["waves_per_row"] == 0
                assert v["waves_per_block"] * 64 <= 1024
            assert max(v["max_n"] for v in vs) == cap
            picked = [v for v in vs if not v["alternative"]]
            # the dispatched general entries cover 1..reach in ascending caps
            general = [v["max_n"] for v in picked if not v["exact"]]
            assert general == sorted(general)
            reach = general[-1]
            for N in (1, 7, 255, 256, 257, 768, 1000, 4096, reach, cap):
                i = rk.variant_pick(op, dt, N)
                assert i >= 0 and not vs[i]["alternative"]
                assert vs[i]["max_n"] == N if vs[i]["exact"] else vs[i]["max_n"] >= N
                if not vs[i]["exact"]:  # the smallest general tile that holds N
                    assert vs[i]["max_n"] == min(c for c in general if c >= N)
            assert rk.variant_pick(op, dt, cap + 1) == -1
            if reach < cap:  # between the two, rows stay in memory
                assert rk.variant_pick(op, dt, reach + 1) == -1
                assert rk.variant_pick(op, dt, cap - 1) == -1
            # exact entries are taken when they fit; rows of that length at
            # other offsets need a general tile that holds them (a dispatched
            # one up to the general reach, else an alternative of that size)
            caps = {v["max_n"] for v in vs if not v["exact"]}
            for v in picked:
                if v["exact"]:
                    assert vs[rk.variant_pick(op, dt, v["max_n"])]["exact"]
                    assert v["max_n"] <= reach or v["max_n"] in caps
            # an alternative is never picked
            for v in vs:
                if v["alternative"]:
                    assert rk.variant_pick(op, dt, v["max_n"]) != v["index"]


def test_variant_entry_points_reject(lib):
    n = lib.rk__variant_count(0, F32)
    assert lib.rk__variant_count(5, F32) == 0 and lib.rk__variant_count(0, 9) == 0
    assert lib.rk__variant_info(0, F32, n, None, None, None, None, None, None, None) == INVALID
    assert lib.rk__softmax_variant(n, A, B, 4, 8, 8, 8, F32, None) == INVALID
    assert lib.rk__softmax_variant(-2, A, B, 4, 8, 8, 8, F32, None) == INVALID
    assert lib.rk__layernorm_gelu_variant(0, A, A + 0x80000, A + 0x90000, B, 4, 8, 8, 8, 0.0,
                                          F32, 0, None) == INVALID
    assert lib.rk__layernorm_gelu_variant(0, A, A + 0x80000, A + 0x90000, B, 4, 8, 8, 8, 1e-5,
                                          F32, 3, None) == INVALID
    n = lib.rk__variant_count(rk.RK_OP_RMSNORM, F32)
    assert n == lib.rk__variant_count(rk.RK_OP_RESIDUAL_RMSNORM, F32) > 0
    assert lib.rk__rmsnorm_variant(n, A, A + 0x80000, B, 4, 8, 8, 8, 1e-5, F32, None) == INVALID
    assert lib.rk__rmsnorm_variant(-2, A, A + 0x80000, B, 4, 8, 8, 8, 1e-5, F32, None) == INVALID
    assert lib.rk__residual_rmsnorm_variant(n, A, C, A + 0x80000, B, D, 4, 8, 8, 8, 8, 8, 1e-5,
                                            F32, None) == INVALID
    assert lib.rk__residual_rmsnorm_variant(0, A, C, A + 0x80000, B, B, 4, 8, 8, 8, 8, 8, 1e-5,
                                            F32, None) == INVALID


def test_product_path_has_no_oracle_or_cpu_fallback():
    pkg = os.path.join(ROOT, "row_wise_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if not path.endswith((".py", ".hip", ".cpp", ".h")):
            continue
        text = open(path).read()
        assert "import oracle" not in text and "from oracle" not in text, path
        assert "liboracle" not in text, path
        if path.endswith(".py"):
            for fn in ("torch.softmax", "F.softmax", "layer_norm(", "F.gelu", ".softmax(",
                       "rms_norm", ".rsqrt("):
                assert fn not in text, (path, fn)
