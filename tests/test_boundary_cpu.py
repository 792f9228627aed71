"""The C-ABI library without a GPU: it loads, exports every declared symbol, and every
invalid argument is rejected with its status before any HIP call is made.

The pointers used here are fake (never dereferenced): validation is pure host
arithmetic, so these calls return before touching the device.
"""

import ctypes
import os
import re

import pytest

from exact_attention_35_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(capi.library_path()),
                                reason="libfa.so not built (run __graft_entry__.build())")

BASE = 0x7f0000000000  # fake, 256-byte aligned device addresses


def _declared_functions():
    text = "".join(open(os.path.join(ROOT, "include", f)).read()
                   for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = capi.lib()
    names = _declared_functions()
    assert set(names) == set(capi.EXPORTED)
    for n in names:
        assert getattr(L, n) is not None


def test_version_and_status_strings():
    text = open(HEADER).read()
    ver = int(re.search(r"#define FA_VERSION (\d+)", text).group(1))
    assert capi.fa_version() == ver
    codes = dict(re.findall(r"(FA_(?:OK|ERR_[A-Z]+))\s*=\s*(-?\d+)", text))
    assert {k: int(v) for k, v in codes.items()} == capi.STATUS
    msgs = {capi.fa_status_string(c) for c in capi.STATUS.values()}
    assert len(msgs) == len(capi.STATUS)
    assert capi.fa_status_string(12345) == "unknown status"


class Call:
    """One fa_fwd / fa_fwd_ex call with fake pointers and contiguous strides."""

    def __init__(self, B=2, H=3, N=100, d=128, dv=128, dtype=capi.FA_BF16, mask=0, bias=False,
                 lse=True):
        es = 2 if dtype == capi.FA_BF16 else 4
        self.B, self.H, self.N, self.d, self.dv, self.dtype, self.mask = B, H, N, d, dv, dtype, mask
        gap = 1 << 32
        self.q = BASE
        self.k = BASE + gap
        self.v = BASE + 2 * gap
        self.out = BASE + 3 * gap
        self.lse = BASE + 4 * gap if lse else 0
        self.bias = BASE + 5 * gap if bias else 0
        s = capi.FaStrides()
        s.q[:] = [H * N * d, N * d, d]
        s.k[:] = [H * N * d, N * d, d]
        s.v[:] = [H * N * dv, N * dv, dv]
        s.out[:] = [H * N * dv, N * dv, dv]
        s.bias[:] = [0, N * N, N]
        s.lse[:] = [H * N, N]
        self.s = s
        self.es = es

    def args(self):
        vp = ctypes.c_void_p
        return (vp(self.q), vp(self.k), vp(self.v), vp(self.bias), self.mask, vp(self.out),
                vp(self.lse), self.B, self.H, self.N, self.d, self.dv, ctypes.byref(self.s),
                self.dtype, vp(0))

    def fwd(self):
        return capi.lib().fa_fwd(*self.args())

    def fwd_ex(self, ws=0, nbytes=0):
        return capi.lib().fa_fwd_ex(*self.args(), ctypes.c_void_p(ws), nbytes)


S = capi.STATUS


@pytest.mark.parametrize("mutate,expected", [
    (lambda c: setattr(c, "dtype", 3), "FA_ERR_DTYPE"),
    (lambda c: setattr(c, "mask", 2), "FA_ERR_MASK"),
    (lambda c: setattr(c, "d", 257), "FA_ERR_SHAPE"),
    (lambda c: setattr(c, "dv", 0), "FA_ERR_SHAPE"),
    (lambda c: setattr(c, "B", -1), "FA_ERR_SHAPE"),
    (lambda c: setattr(c, "N", 1 << 31), "FA_ERR_SHAPE"),
    (lambda c: setattr(c, "q", 0), "FA_ERR_NULL"),
    (lambda c: setattr(c, "k", 0), "FA_ERR_NULL"),
    (lambda c: setattr(c, "v", 0), "FA_ERR_NULL"),
    (lambda c: setattr(c, "out", 0), "FA_ERR_NULL"),
    (lambda c: c.s.q.__setitem__(2, -128), "FA_ERR_STRIDE"),
    (lambda c: c.s.out.__setitem__(2, 64), "FA_ERR_STRIDE"),       # rows overlap (dv=128)
    (lambda c: c.s.lse.__setitem__(1, 50), "FA_ERR_STRIDE"),       # heads overlap (N=100)
    (lambda c: setattr(c, "q", BASE + 1), "FA_ERR_ALIGN"),         # not 2-byte aligned (bf16)
    (lambda c: setattr(c, "out", c.out + 3), "FA_ERR_ALIGN"),
    (lambda c: setattr(c, "lse", c.lse + 2), "FA_ERR_ALIGN"),
    (lambda c: setattr(c, "out", c.q), "FA_ERR_ALIAS"),
    (lambda c: setattr(c, "out", c.v + 256), "FA_ERR_ALIAS"),
    (lambda c: setattr(c, "lse", c.out + 1024), "FA_ERR_ALIAS"),
    (lambda c: setattr(c, "lse", c.k), "FA_ERR_ALIAS"),
])
def test_invalid_arguments_rejected_before_launch(mutate, expected):
    c = Call()
    mutate(c)
    assert c.fwd() == S[expected]
    assert c.fwd_ex() == S[expected]


def test_bias_aliasing_and_alignment():
    c = Call(bias=True)
    c.bias = c.out
    assert c.fwd() == S["FA_ERR_ALIAS"]
    c = Call(bias=True)
    c.bias = c.bias + 2
    assert c.fwd() == S["FA_ERR_ALIGN"]
    c = Call(bias=True)
    c.lse = c.bias + 4096
    assert c.fwd() == S["FA_ERR_ALIAS"]


@pytest.mark.parametrize("B,H,N", [(0, 4, 128), (2, 0, 128), (2, 4, 0)])
def test_zero_size_is_ok_without_pointers(B, H, N):
    c = Call(B=B, H=H, N=N)
    c.q = c.k = c.v = c.out = c.lse = 0
    assert c.fwd() == S["FA_OK"]
    assert c.fwd_ex() == S["FA_OK"]


def test_alignment_is_per_element_size_and_other_layouts_are_valid():
    # fp32 needs 4-byte aligned bases; 16-byte alignment, odd widths and fp16 only select
    # the general kernel (valid arguments reach the device check, which fails without a
    # gfx950 GPU)
    ok = (S["FA_ERR_DEVICE"], S["FA_OK"])
    c = Call(dtype=capi.FA_F32, d=64, dv=64)
    c.out = c.q + (1 << 30)
    c.s.q[2] = 66          # 264-byte rows: not 16-byte aligned, still valid
    c.s.q[1] = 66 * c.N
    c.s.q[0] = 66 * c.N * c.H
    assert c.fwd() in ok
    c.q += 2               # 2-byte aligned fp32 base: invalid
    assert c.fwd() == S["FA_ERR_ALIGN"]
    for kw in (dict(d=96), dict(dv=40), dict(d=1, dv=256), dict(dtype=capi.FA_F16)):
        c = Call(**kw)
        assert c.fwd() in ok, kw
    c = Call()
    c.q += 2               # bf16 base 2-byte aligned: the general kernel takes it
    assert c.fwd() in ok
    c = Call()
    c.s.k[2] = 1 << 24     # a key row stride the matrix-core kernel cannot address
    c.s.k[1] = c.s.k[2] * c.N
    c.s.k[0] = c.s.k[1] * c.H
    c.v = c.k + c.s.k[0] * c.B * 2  # keep v past the strided k
    c.out = c.v + (1 << 32)
    c.lse = c.out + (1 << 32)
    assert c.fwd() in ok


def test_workspace_size_invalid_is_zero():
    L = capi.lib()
    assert L.fa_fwd_workspace_size(1, 1, 8192, 96, 128, capi.FA_BF16, 1) == 0
    assert L.fa_fwd_workspace_size(1, 1, 0, 128, 128, capi.FA_BF16, 1) == 0
    assert L.fa_fwd_workspace_size(1, 1, 64, 128, 128, 7, 1) == 0


def test_python_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(capi.FaError):
        capi.fa_fwd(q, q, q[:, :, :8])
    with pytest.raises(capi.FaError):
        capi.fa_fwd(q, q.float(), q)
    with pytest.raises(capi.FaError):
        capi.fa_fwd(q.transpose(-1, -2).contiguous().transpose(-1, -2), q, q)
    with pytest.raises(capi.FaError):
        capi.fa_fwd(q.double(), q.double(), q.double())


def _qk_call(c, Nq, Nk, k=None, v=None):
    vp = ctypes.c_void_p
    return capi.lib().fa_fwd_qk(vp(c.q), vp(c.k if k is None else k), vp(c.v if v is None else v), vp(c.bias),
                                c.mask, vp(c.out), vp(c.lse), c.B, c.H, Nq, Nk, c.d, c.dv, None, c.dtype, vp(0))


def test_rectangular_entry_validation():
    c = Call()
    assert _qk_call(c, -1, 100) == S["FA_ERR_SHAPE"]
    assert _qk_call(c, 100, -1) == S["FA_ERR_SHAPE"]
    assert _qk_call(c, 100, 1 << 31) == S["FA_ERR_SHAPE"]
    assert _qk_call(c, 100, 50, k=0) == S["FA_ERR_NULL"]
    # no query rows: nothing to do; no keys: k and v may be NULL (reaches the device check)
    assert _qk_call(c, 0, 50) == S["FA_OK"]
    assert _qk_call(c, 10, 0, k=0, v=0) in (S["FA_ERR_DEVICE"], S["FA_OK"])
    # out over k is caught with the key extent (N_k rows), not the query extent
    c2 = Call(N=10)
    c2.out = c2.k + 29440  # inside the 20-row extent of k (30720 bytes), past a 10-row one (28160)
    assert _qk_call(c2, 10, 20) == S["FA_ERR_ALIAS"]
    assert capi.lib().fa_fwd_qk_workspace_size(1, 1, 1, 100, 96, 128, capi.FA_BF16, 1) == 0
