"""The gradient entry points (include/fa_bwd.h) without a GPU: every invalid argument
is rejected with its status before any HIP call is made (fake, never dereferenced
pointers), and the workspace size follows the row-statistics layout."""

import ctypes
import os

import pytest

from exact_attention_35_amd import capi

pytestmark = pytest.mark.skipif(not os.path.exists(capi.library_path()),
                                reason="libfa.so not built (run __graft_entry__.build())")

BASE = 0x7f0000000000
S = capi.STATUS
NAMES = ("q", "k", "v", "out", "grad_out", "grad_q", "grad_k", "grad_v")


class BwdCall:
    def __init__(self, B=2, H=3, N=100, d=128, dv=128, dtype=capi.FA_BF16, mask=0, bias=False):
        self.B, self.H, self.N, self.d, self.dv, self.dtype, self.mask = B, H, N, d, dv, dtype, mask
        gap = 1 << 32
        self.ptr = {n: BASE + i * gap for i, n in enumerate(NAMES)}
        self.lse = BASE + 8 * gap
        self.bias = BASE + 9 * gap if bias else 0
        s = capi.FaBwdStrides()
        for n in NAMES:
            w = d if n in ("q", "k", "grad_q", "grad_k") else dv
            getattr(s, n)[:] = [H * N * w, N * w, w]
        s.bias[:] = [0, N * N, N]
        s.lse[:] = [H * N, N]
        self.s = s

    def args(self):
        vp = ctypes.c_void_p
        p = self.ptr
        return (vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["out"]), vp(self.lse), vp(p["grad_out"]),
                vp(self.bias), self.mask, vp(p["grad_q"]), vp(p["grad_k"]), vp(p["grad_v"]),
                self.B, self.H, self.N, self.d, self.dv, ctypes.byref(self.s), self.dtype, vp(0))

    def bwd(self):
        return capi.lib().fa_bwd(*self.args())

    def bwd_ex(self):
        return capi.lib().fa_bwd_ex(*self.args(), ctypes.c_void_p(0), 0)


def _set(name, value):
    return lambda c: c.ptr.__setitem__(name, value)


@pytest.mark.parametrize("mutate,expected", [
    (lambda c: setattr(c, "dtype", capi.FA_F32), "FA_ERR_DTYPE"),
    (lambda c: setattr(c, "dtype", 3), "FA_ERR_DTYPE"),
    (lambda c: setattr(c, "dtype", 5), "FA_ERR_DTYPE"),
    (lambda c: setattr(c, "mask", 3), "FA_ERR_MASK"),
    (lambda c: setattr(c, "d", 80), "FA_ERR_SHAPE"),
    (lambda c: setattr(c, "H", -2), "FA_ERR_SHAPE"),
    (lambda c: setattr(c, "lse", 0), "FA_ERR_NULL"),
    (_set("grad_out", 0), "FA_ERR_NULL"),
    (_set("out", 0), "FA_ERR_NULL"),
    (_set("grad_v", 0), "FA_ERR_NULL"),
    (lambda c: c.s.grad_q.__setitem__(2, 64), "FA_ERR_STRIDE"),   # dQ rows overlap
    (lambda c: c.s.grad_out.__setitem__(0, -1), "FA_ERR_STRIDE"),
    (lambda c: c.s.q.__setitem__(2, 1 << 24), "FA_ERR_STRIDE"),   # tile offsets overflow
    (lambda c: c.s.grad_out.__setitem__(2, 1 << 24), "FA_ERR_STRIDE"),
    (_set("grad_k", BASE + 7 * (1 << 32) + 8), "FA_ERR_ALIGN"),
    (lambda c: c.s.out.__setitem__(2, 132), "FA_ERR_ALIGN"),
    (lambda c: setattr(c, "lse", c.lse + 2), "FA_ERR_ALIGN"),
    (_set("grad_q", BASE), "FA_ERR_ALIAS"),                       # dQ over q
    (_set("grad_v", BASE + 6 * (1 << 32) + 4096), "FA_ERR_ALIAS"),  # dV over dK
    (lambda c: setattr(c, "lse", c.ptr["grad_k"] + 512), "FA_ERR_ALIAS"),
])
def test_invalid_gradient_arguments_rejected(mutate, expected):
    c = BwdCall()
    mutate(c)
    assert c.bwd() == S[expected]
    assert c.bwd_ex() == S[expected]


def test_bias_overlapping_a_gradient_is_rejected():
    c = BwdCall(bias=True)
    c.bias = c.ptr["grad_q"]
    assert c.bwd() == S["FA_ERR_ALIAS"]


def test_zero_size_gradients_need_no_pointers():
    c = BwdCall(N=0)
    c.ptr = {n: 0 for n in NAMES}
    c.lse = 0
    assert c.bwd() == S["FA_OK"] and c.bwd_ex() == S["FA_OK"]


def test_gradient_workspace_size_of_invalid_arguments_is_zero():
    L = capi.lib()
    assert L.fa_bwd_workspace_size(1, 1, 8192, 128, 128, capi.FA_F32, 1) == 0
    assert L.fa_bwd_workspace_size(1, 1, 8192, 96, 128, capi.FA_BF16, 1) == 0
    assert L.fa_bwd_workspace_size(1, 1, 0, 128, 128, capi.FA_BF16, 0) == 0
    assert L.fa_bwd_workspace_size(1, 1, 100, 128, 128, capi.FA_BF16, 5) == 0
