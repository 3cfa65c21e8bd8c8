"""Host-only checks of libmhc.so: it loads, exports every entry point that
include/mhc.h declares, and rejects invalid arguments on the host before anything
is enqueued (no GPU is touched by any call here: every call fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")
LIBP = os.path.join(ROOT, "manifold_constrained_residuals_amd", "libmhc.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIBP):
        import manifold_constrained_residuals_amd.build as b
        b.build()
    return ctypes.CDLL(LIBP)


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    L.mhc_status_str.restype = ctypes.c_char_p
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8, 12345):
        s = L.mhc_status_str(st)
        assert s and len(s) > 5
    assert L.mhc_abi_version() == 2


def test_workspace_sizes(L):
    L.mhc_workspace_size.restype = ctypes.c_size_t
    L.mhc_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    bwd = L.mhc_workspace_size(1, 16384, 4, 4096, 1)
    assert bwd >= 16384 * 4 * 4096 * 24 // 64 * 0 + 16384 * 24 * 4
    assert L.mhc_workspace_size(3, 16384, 4, 4096, 1) == bwd
    assert L.mhc_workspace_size(1, 0, 4, 4096, 1) == 0      # invalid T
    assert L.mhc_workspace_size(1, 16, 3, 4096, 1) == 0     # invalid n
    assert L.mhc_workspace_size(1, 16, 4, 12, 1) == 0       # C % 8
    assert L.mhc_workspace_size(1, 16, 4, 4096, 9) == 0     # dtype


def _pre(L, T, n, C, dt, X, H, u):
    f = L.mhc_pre
    f.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return f(T, n, C, dt, X, H, u, None)


def test_validation_errors_before_launch(L):
    A = 0x10000  # never dereferenced: every call below fails validation first
    assert _pre(L, 0, 4, 64, 1, A, A, A) == -2          # T < 1
    assert _pre(L, 8, 3, 64, 1, A, A, A) == -2          # n not in {1, 4}
    assert _pre(L, 8, 4, 60, 1, A, A, A) == -2          # C % 8 != 0
    assert _pre(L, 8, 4, 64, 5, A, A, A) == -4          # dtype
    assert _pre(L, 8, 4, 64, 1, None, A, A) == -1       # NULL
    assert _pre(L, 8, 4, 64, 1, A + 4, A, A) == -3      # misaligned
    f = L.mhc_sinkhorn
    f.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert f(8, 4, A, 16, 0, A, None) == -5             # iters < 1
    assert f(8, 4, A, 15, 20, A, None) == -2            # ld < n*n
    g = L.mhc_coeffs_bwd
    vp = ctypes.c_void_p
    g.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int] + [vp] * 17 + [vp, ctypes.c_size_t, vp]
    alpha = (ctypes.c_float * 3)(1, 1, 1)
    args = [A] * 3 + [ctypes.addressof(alpha)] + [A] * 8 + [A, A, A, A, A]
    assert g(64, 4, 256, 1, *args, A, 16, None) == -6   # workspace too small
    assert g(64, 4, 256, 1, *args, None, 0, None) == -6  # workspace missing


def test_cross_layer_entries_validate(L):
    A = 0x10000
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.mhc_workspace_size.restype = ctypes.c_size_t
    L.mhc_workspace_size.argtypes = [i32, i64, i32, i64, i32]
    ws = L.mhc_workspace_size(4, 16384, 4, 4096, 1)
    assert ws >= 4 * 4096 * 48 * 2 + 16384 * 32 * 4            # split W' + one partial set
    assert L.mhc_workspace_size(4, 16384, 4, 4096, 0) == 0  # fp32: not supported
    assert L.mhc_workspace_size(4, 16384, 1, 4096, 1) == 0  # n = 1: not supported
    f = L.mhc_post_res_next
    f.argtypes = [i64, i32, i64, i32] + [vp] * 7 + [vp, ctypes.c_size_t, vp]
    ok = [A] * 7
    assert f(64, 4, 256, 0, *ok, A, 1 << 30, None) == -4     # fp32 storage
    assert f(64, 1, 256, 1, *ok, A, 1 << 30, None) == -2     # n = 1
    assert f(64, 4, 264, 1, *ok, A, 1 << 30, None) == -2     # C % 64 != 0
    assert f(64, 4, 256, 1, *([A] * 6 + [None]), A, 1 << 30, None) == -1
    assert f(64, 4, 256, 1, *ok, A, 16, None) == -6          # workspace too small
    g = L.mhc_fwd_pre_next
    g.argtypes = [i64, i32, i64, i32, vp, ctypes.c_float, vp, vp, i32] + [vp] * 8 + [vp, ctypes.c_size_t, vp]
    alpha = (ctypes.c_float * 3)(1, 1, 1)
    outs = [A] * 6 + [None]                                  # z .. u, proj
    assert g(64, 4, 256, 1, A, 1e-6, A, ctypes.addressof(alpha), 0, None, *outs, A, 1 << 30, None) == -5
    assert g(64, 4, 256, 1, A, 1e-6, A, None, 20, None, *outs, A, 1 << 30, None) == -1
    assert g(64, 4, 256, 1, A, 1e-6, A, ctypes.addressof(alpha), 20, A + 4, *outs, A, 1 << 30, None) == -3
    assert g(64, 4, 256, 1, A, 1e-6, A, ctypes.addressof(alpha), 20, None, *outs, None, 0, None) == -6


def test_post_res_fwd_pre_validates(L):
    """mhc_post_res_fwd_pre rejects bad arguments before anything is enqueued: NULL
    required pointers, an output overlapping an input (X_out on X or F_out, u on X, the
    next layer's maps on this layer's), iters < 1, a non-finite alpha, a short
    workspace."""
    A, B = 0x10000000, 0x20000000           # inputs at A, outputs at B: disjoint ranges
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.mhc_workspace_size.restype = sz
    L.mhc_workspace_size.argtypes = [i32, i64, i32, i64, i32]
    T, n, C = 64, 4, 1024
    ws = L.mhc_workspace_size(2, T, n, C, 1)
    assert ws > 0
    f = L.mhc_post_res_fwd_pre
    f.argtypes = ([i64, i32, i64, i32] + [vp] * 6 + [f32, vp, vp, vp, i32] + [vp] * 8 +
                  [vp, sz, vp])
    alpha = (ctypes.c_float * 3)(1, 1, 1)
    pa = ctypes.addressof(alpha)

    def call(X=A, F=A, Hr=A, Hp=A, Xo=B, g=A, W=A, b=A, al=pa, it=20, zin=None, Hrn=B, Hpn=B,
             u=B, proj=None, w=A, wb=ws):
        return f(T, n, C, 1, X, F, Hr, Hp, Xo, g, 1e-6, W, b, al, it, zin, B, B, B, Hpn, Hrn, u,
                 proj, w, wb, None)

    assert call(X=None) == -1
    assert call(F=None) == -1
    assert call(Hrn=None) == -1
    assert call(Xo=A) == -2                                  # X_out is X
    assert call(Xo=A + 4096, X=A + (1 << 24)) == -2          # X_out overlaps F_out
    assert call(u=A + 64) == -2                              # u overlaps X
    assert call(Hrn=A) == -2                                 # H_res_next is H_res
    assert call(Hpn=A + 16) == -2                            # H_post_next overlaps H_post
    assert call(it=0) == -5
    assert call(al=None) == -1
    assert call(wb=ws - 256) == -6
    assert call(w=None) == -6
    bad = (ctypes.c_float * 3)(1, float("nan"), 1)
    assert call(al=ctypes.addressof(bad)) == -8


def test_alpha_bwd_validates(L):
    A = 0x10000
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.mhc_workspace_size.restype = ctypes.c_size_t
    L.mhc_workspace_size.argtypes = [i32, i64, i32, i64, i32]
    ws = L.mhc_workspace_size(5, 16384, 4, 4096, 1)
    assert ws >= 3 * 8 and ws == L.mhc_workspace_size(5, 1, 8, 8, 0)
    f = L.mhc_alpha_bwd
    f.argtypes = [i64, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    assert f(64, 3, A, A, A, A, ws, None) == -2
    assert f(0, 4, A, A, A, A, ws, None) == -2
    assert f(64, 4, None, A, A, A, ws, None) == -1
    assert f(64, 4, A, None, A, A, ws, None) == -1
    assert f(64, 4, A, A, A + 4, A, ws, None) == -3
    assert f(64, 4, A, A, A, A, ws - 8, None) == -6
    assert f(64, 4, A, A, A, None, ws, None) == -6


def test_non_finite_alpha_rejected_by_every_entry(L):
    """Every single-layer entry that takes alpha rejects a NaN or an infinite entry
    with MHC_ERR_VALUE before anything is enqueued."""
    A = 0x10000
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.mhc_workspace_size.restype = sz
    L.mhc_workspace_size.argtypes = [i32, i64, i32, i64, i32]
    T, n, C = 64, 4, 256
    wsf = L.mhc_workspace_size(2, T, n, C, 1)
    wsb = L.mhc_workspace_size(3, T, n, C, 1)
    wsn = L.mhc_workspace_size(4, T, n, C, 1)
    L.mhc_status_str.restype = ctypes.c_char_p
    assert b"alpha" in L.mhc_status_str(-8)
    for bad in ((0.5, float("nan"), 0.5), (float("inf"), 0.5, 0.5), (0.5, 0.5, float("-inf"))):
        a = (ctypes.c_float * 3)(*bad)
        pa = ctypes.addressof(a)
        f = L.mhc_coeffs
        f.argtypes = [i64, i32, i64, i32, vp, vp, f32, vp, vp, vp] + [vp] * 5 + [vp, sz, vp]
        assert f(T, n, C, 1, A, A, 1e-6, A, A, pa, A, A, A, A, None, A, wsf, None) == -8
        f = L.mhc_fwd_pre
        f.argtypes = [i64, i32, i64, i32, vp, vp, f32, vp, vp, vp, i32] + [vp] * 8 + [vp, sz, vp]
        assert f(T, n, C, 1, A, A, 1e-6, A, A, pa, 20, None, A, A, A, A, A, A, None, A, wsf,
                 None) == -8
        f = L.mhc_fwd_pre_next
        f.argtypes = [i64, i32, i64, i32, vp, f32, vp, vp, i32] + [vp] * 8 + [vp, sz, vp]
        assert f(T, n, C, 1, A, 1e-6, A, pa, 20, None, A, A, A, A, A, A, None, A, wsn, None) == -8
        f = L.mhc_coeffs_bwd
        f.argtypes = [i64, i32, i64, i32] + [vp] * 17 + [vp, sz, vp]
        assert f(T, n, C, 1, A, A, A, pa, *([A] * 13), A, wsb, None) == -8
        f = L.mhc_bwd_pre
        f.argtypes = [i64, i32, i64, i32] + [vp] * 14 + [i32] + [vp] * 7 + [vp, sz, vp]
        assert f(T, n, C, 1, A, A, A, A, A, pa, *([A] * 8), 20, None, *([A] * 5), None, A, wsb,
                 None) == -8
        f = L.mhc_bwd_pre_from_dh
        f.argtypes = [i64, i32, i64, i32] + [vp] * 15 + [i32] + [vp] * 6 + [vp, sz, vp]
        assert f(T, n, C, 1, A, A, A, A, A, pa, *([A] * 9), 20, None, *([A] * 4), None, A, wsb,
                 None) == -8


def test_stack_block_size_and_workspace(L):
    L.mhc_stack_block_size.argtypes = [ctypes.c_int]
    L.mhc_stack_block_size.restype = ctypes.c_int
    for nl in range(1, 130):
        costs = [(-(-nl // b) + b - 1, b) for b in range(1, nl + 1)]
        assert L.mhc_stack_block_size(nl) == min(costs)[1], nl
    assert L.mhc_stack_block_size(0) == 0
    f = L.mhc_stack_workspace_size
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    f.restype = ctypes.c_size_t
    sizes = [f(16, b, 4096, 4, 2048, 1) for b in range(1, 17)]
    assert all(s > 0 for s in sizes)
    # one more block buffer of X (bf16 [T][4][C]) per unit of B once the backward dominates
    xb = 4096 * 4 * 2048 * 2
    assert sizes[15] - sizes[14] == xb
    assert f(16, 0, 4096, 4, 2048, 1) == 0 and f(16, 17, 4096, 4, 2048, 1) == 0
    assert f(0, 1, 4096, 4, 2048, 1) == 0 and f(4, 2, 4096, 3, 2048, 1) == 0


def test_stack_entries_validate(L):
    A = 0x10000
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f = L.mhc_stack_forward
    f.argtypes = [i32, i32, i64, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, i32,
                  vp, vp, vp, ctypes.c_size_t, vp]
    arr = (vp * 4)(A, A, A, A)
    bad = (vp * 4)(A, A, None, A)
    mis = (vp * 4)(A, A, A + 8, A)
    al = (ctypes.c_float * 12)(*([0.5] * 12))
    aln = (ctypes.c_float * 12)(*([0.5] * 11 + [float("nan")]))
    P = ctypes.addressof
    ok = lambda **kw: dict(dict(L=4, B=2, T=64, n=4, C=256, dt=1, X0=A, g=P(arr), W=P(arr), b=P(arr),
                                al=P(al), F=P(arr), u=None, it=20, Xs=P(arr), XL=A + 0x100, ws=A,
                                wb=1 << 40), **kw)
    call = lambda d: f(d["L"], d["B"], d["T"], d["n"], d["C"], d["dt"], d["X0"], d["g"], d["W"], d["b"],
                       d["al"], d["F"], d["u"], 1e-6, d["it"], d["Xs"], d["XL"], d["ws"], d["wb"], None)
    assert call(ok(B=0)) == -2 and call(ok(B=5)) == -2 and call(ok(L=0)) == -2
    assert call(ok(n=3)) == -2 and call(ok(dt=7)) == -4 and call(ok(it=0)) == -5
    assert call(ok(W=P(bad))) == -1 and call(ok(F=None)) == -1 and call(ok(al=None)) == -1
    assert call(ok(b=P(mis))) == -3 and call(ok(u=P(mis))) == -3
    assert call(ok(al=P(aln))) == -8
    assert call(ok(XL=A)) == -2                       # X_L is one of the saved buffers
    assert call(ok(wb=16)) == -6
    g = L.mhc_stack_backward
    g.argtypes = [i32, i32, i64, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                  vp, ctypes.c_size_t, vp]
    args = lambda du=P(arr), dW=P(arr), wb=1 << 40, B=2: g(4, B, 64, 4, 256, 1, P(arr), P(arr), P(arr),
                                                          P(arr), P(al), P(arr), du, 20, A, A, dW,
                                                          P(arr), None, A, wb, None)
    assert args(du=None) == -1 and args(dW=P(bad)) == -1 and args(wb=16) == -6 and args(B=9) == -2


def test_split_backward_entries_validate(L):
    A = 0x10000
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f = L.mhc_post_res_bwd_pre
    f.argtypes = [i64, i32, i64, i32] + [vp] * 10 + [vp]
    ok = [A] * 10
    assert f(0, 4, 256, 1, *ok, None) == -2                    # T < 1
    assert f(64, 4, 256, 7, *ok, None) == -4                   # dtype
    assert f(64, 4, 256, 1, A, None, *([A] * 8), None) == -1   # du NULL
    assert f(64, 4, 256, 1, *([A] * 9 + [None]), None) == -1   # dH_pre NULL
    assert f(64, 4, 256, 1, *([A] * 9 + [A + 4]), None) == -3  # misaligned dH_pre
    L.mhc_workspace_size.restype = ctypes.c_size_t
    L.mhc_workspace_size.argtypes = [i32, i64, i32, i64, i32]
    ws = L.mhc_workspace_size(3, 64, 4, 256, 1)
    g = L.mhc_bwd_pre_from_dh
    g.argtypes = [i64, i32, i64, i32] + [vp] * 15 + [i32] + [vp] * 6 + [vp, ctypes.c_size_t, vp]
    alpha = (ctypes.c_float * 3)(1, 1, 1)
    ins = [A, A, A, A, A, ctypes.addressof(alpha)] + [A] * 9     # dX_out .. dH_post
    outs = [A] * 5 + [None]                                         # z_res_in, dX, dW, dbias, dz, dgamma
    assert g(64, 4, 256, 1, *ins, 0, *outs, A, ws, None) == -5     # iters
    assert g(64, 4, 256, 1, *ins[:5], None, *ins[6:], 20, *outs, A, ws, None) == -1   # alpha
    assert g(64, 4, 256, 1, *ins[:12], None, *ins[13:], 20, *outs, A, ws, None) == -1  # dH_pre
    assert g(64, 4, 256, 1, *ins, 20, *outs, A, ws - 256, None) == -6                  # workspace
    assert g(64, 4, 256, 1, *ins, 20, *outs, None, ws, None) == -6


def test_noalloc_forward_validates(L):
    """mhc_fwd_pre_noalloc rejects sizes whose scratch exceeds its built-in array
    (MHC_ERR_SCRATCH), and the usual argument errors, before touching any device."""
    A = 0x10000
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    f = L.mhc_fwd_pre_noalloc
    f.argtypes = [i64, i32, i64, i32, vp, vp, f32, vp, vp, vp, i32] + [vp] * 8 + [vp]
    L.mhc_workspace_size.restype = sz
    L.mhc_workspace_size.argtypes = [i32, i64, i32, i64, i32]
    al = (ctypes.c_float * 3)(1, 1, 1)
    pa = ctypes.addressof(al)
    outs = [A] * 7 + [None]                       # z, rms, H_pre, H_post, H_res, u, proj
    big = 262144
    assert L.mhc_workspace_size(2, big, 4, 4096, 1) > 64 << 20
    assert f(big, 4, 4096, 1, A, A, 1e-6, A, A, pa, 20, None, *outs[1:], None) == -9
    assert f(64, 4, 256, 1, None, A, 1e-6, A, A, pa, 20, None, *outs[1:], None) == -1
    bad = (ctypes.c_float * 3)(1, float("nan"), 1)
    assert f(64, 4, 256, 1, A, A, 1e-6, A, A, ctypes.addressof(bad), 20, None, *outs[1:], None) == -8
    assert f(64, 4, 256, 1, A, A, 1e-6, A, A, pa, 0, None, *outs[1:], None) == -5
    L.mhc_status_str.restype = ctypes.c_char_p
    assert b"scratch" in L.mhc_status_str(-9)


def test_nonfinite_status_string(L):
    """MHC_ERR_NONFINITE (-10), returned only under MHC_CHECK_FINITE, has its message."""
    L.mhc_status_str.restype = ctypes.c_char_p
    assert b"NONFINITE" in L.mhc_status_str(-10)
