"""Thin Python binding of the C ABI in include/*.h (argument marshalling only).

Every function here has the name of the C entry point it wraps. Tensors are torch
tensors in logical [B, H, N, *] layout with any strides whose innermost axis is
contiguous; pointers, element strides and torch's current HIP stream are passed
through unchanged. All arithmetic runs in libfa.so's HIP kernels; if the library is
not built, every call raises — there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "FaError", "FA_OK", "FA_F32", "FA_BF16", "FA_F16", "FA_MASK_NONE", "FA_MASK_CAUSAL",
    "STATUS", "lib", "library_path", "fa_fwd", "fa_fwd_ex", "fa_fwd_workspace_size",
    "fa_status_string", "fa_version", "fa_shutdown", "fa_plan_describe", "make_strides", "FaStrides",
    "FaPlanInfo", "EXPORTED", "fa_bwd", "fa_bwd_ex", "fa_bwd_workspace_size", "FaBwdStrides",
    "fa_fwd_qk", "fa_fwd_qk_ex", "fa_fwd_qk_workspace_size", "fa_plan_describe_qk", "fa_fwd_qk_noalloc",
    "fa_probe_copy", "fa_probe_mfma", "fa_probe_mfma_flops", "fa_probe_timer_arm", "fa_probe_timer_read",
    "FA_PROBE_TIMER_MAX", "fa_probe_issue", "fa_probe_read", "fa_probe_lds", "fa_probe_tile",
]

FA_OK = 0
FA_F32 = 0
FA_BF16 = 1
FA_F16 = 2
FA_MASK_NONE = 0
FA_MASK_CAUSAL = 1
STATUS = {
    "FA_OK": 0, "FA_ERR_NULL": -1, "FA_ERR_SHAPE": -2, "FA_ERR_DTYPE": -3,
    "FA_ERR_MASK": -4, "FA_ERR_STRIDE": -5, "FA_ERR_ALIGN": -6, "FA_ERR_ALIAS": -7,
    "FA_ERR_WORKSPACE": -8, "FA_ERR_LAUNCH": -9, "FA_ERR_DEVICE": -10, "FA_ERR_ALLOC": -11,
}

# every symbol include/*.h declares
EXPORTED = ("fa_fwd", "fa_fwd_ex", "fa_fwd_workspace_size", "fa_status_string",
            "fa_version", "fa_shutdown", "fa_plan_describe", "fa_bwd", "fa_bwd_ex",
            "fa_bwd_workspace_size", "fa_fwd_qk", "fa_fwd_qk_ex", "fa_fwd_qk_workspace_size",
            "fa_plan_describe_qk", "fa_fwd_qk_noalloc", "fa_probe_copy", "fa_probe_mfma",
            "fa_probe_mfma_flops", "fa_probe_timer_arm", "fa_probe_timer_read", "fa_probe_issue",
            "fa_probe_read", "fa_probe_lds", "fa_probe_tile")
FA_PROBE_TIMER_MAX = 4096

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libfa.so")


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fa status {status}: {message}")
        self.status = status


class FaStrides(ctypes.Structure):
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3), ("v", ctypes.c_int64 * 3),
                ("out", ctypes.c_int64 * 3), ("bias", ctypes.c_int64 * 3),
                ("lse", ctypes.c_int64 * 2)]


class FaBwdStrides(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64 * 3) for name in
                ("q", "k", "v", "out", "grad_out", "grad_q", "grad_k", "grad_v", "bias")] + \
               [("lse", ctypes.c_int64 * 2)]


class FaPlanInfo(ctypes.Structure):
    _fields_ = [("split", ctypes.c_int32), ("n_qtiles", ctypes.c_int32), ("qtile_rows", ctypes.c_int32),
                ("key_tile", ctypes.c_int32), ("units", ctypes.c_int32), ("merge_blocks", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("unit_tile_shift", ctypes.c_int32)]


_lib = None


def lib():
    """Load libfa.so (once). Raises if it is missing: the HIP library is the only path."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run exact_attention_35_amd.build.build() "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    fwd_args = [vp, vp, vp, vp, ctypes.c_int, vp, vp, i64, i64, i64, i64, i64,
                ctypes.POINTER(FaStrides), ctypes.c_int, vp]
    L.fa_fwd.argtypes = fwd_args
    L.fa_fwd.restype = ctypes.c_int
    L.fa_fwd_ex.argtypes = fwd_args + [vp, sz]
    L.fa_fwd_ex.restype = ctypes.c_int
    L.fa_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    L.fa_fwd_workspace_size.restype = sz
    qk_args = [vp, vp, vp, vp, ctypes.c_int, vp, vp, i64, i64, i64, i64, i64, i64,
               ctypes.POINTER(FaStrides), ctypes.c_int, vp]
    L.fa_fwd_qk.argtypes = qk_args
    L.fa_fwd_qk.restype = ctypes.c_int
    L.fa_fwd_qk_ex.argtypes = qk_args + [vp, sz]
    L.fa_fwd_qk_ex.restype = ctypes.c_int
    L.fa_fwd_qk_noalloc.argtypes = qk_args
    L.fa_fwd_qk_noalloc.restype = ctypes.c_int
    L.fa_fwd_qk_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    L.fa_fwd_qk_workspace_size.restype = sz
    L.fa_status_string.argtypes = [ctypes.c_int]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = ctypes.c_int
    L.fa_shutdown.argtypes = []
    L.fa_shutdown.restype = None
    L.fa_plan_describe.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(FaPlanInfo), ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    L.fa_plan_describe.restype = ctypes.c_int
    L.fa_plan_describe_qk.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(FaPlanInfo), ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    L.fa_plan_describe_qk.restype = ctypes.c_int
    bwd_args = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, i64,
                ctypes.POINTER(FaBwdStrides), ctypes.c_int, vp]
    L.fa_bwd.argtypes = bwd_args
    L.fa_bwd.restype = ctypes.c_int
    L.fa_bwd_ex.argtypes = bwd_args + [vp, sz]
    L.fa_bwd_ex.restype = ctypes.c_int
    L.fa_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    L.fa_bwd_workspace_size.restype = sz
    L.fa_probe_copy.argtypes = [vp, vp, i64, vp]
    L.fa_probe_copy.restype = ctypes.c_int
    L.fa_probe_mfma.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    L.fa_probe_mfma.restype = ctypes.c_int
    L.fa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.fa_probe_mfma_flops.restype = ctypes.c_double
    L.fa_probe_timer_arm.argtypes = [ctypes.c_int]
    L.fa_probe_timer_arm.restype = ctypes.c_int
    L.fa_probe_timer_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int]
    L.fa_probe_timer_read.restype = ctypes.c_int
    L.fa_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    L.fa_probe_issue.restype = ctypes.c_int
    L.fa_probe_read.argtypes = [vp, i64, vp, ctypes.c_int, vp]
    L.fa_probe_read.restype = ctypes.c_int
    L.fa_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    L.fa_probe_lds.restype = ctypes.c_int
    L.fa_probe_tile.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64, vp, vp, vp]
    L.fa_probe_tile.restype = ctypes.c_int
    _lib = L
    return L


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def fa_version() -> int:
    return int(lib().fa_version())


def fa_shutdown() -> None:
    lib().fa_shutdown()


def fa_plan_describe(B, H, N, d, dv, dtype, causal, compute_units, max_units=4096):
    """The work plan of a problem on a device with `compute_units` CUs (no GPU needed):
    (FaPlanInfo, list of packed unit-table words; empty unless the plan splits)."""
    return fa_plan_describe_qk(B, H, N, N, d, dv, dtype, causal, compute_units, max_units)


def fa_plan_describe_qk(B, H, Nq, Nk, d, dv, dtype, causal, compute_units, max_units=4096):
    """fa_plan_describe for N_q query rows against N_k keys (the plan of fa_fwd_qk)."""
    info = FaPlanInfo()
    table = (ctypes.c_uint32 * max_units)()
    st = lib().fa_plan_describe_qk(B, H, Nq, Nk, d, dv, dtype, FA_MASK_CAUSAL if causal else FA_MASK_NONE,
                                   compute_units, ctypes.byref(info), table, max_units)
    _check(st)
    units = list(table[: min(info.units, max_units)]) if info.split else []
    return info, units


def _check(status: int) -> None:
    if status != FA_OK:
        raise FaError(status, fa_status_string(status))


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.float16:
        return FA_F16
    raise FaError(STATUS["FA_ERR_DTYPE"], f"unsupported dtype {t.dtype}")


def make_strides(q, k, v, out, bias=None, lse=None) -> FaStrides:
    s = FaStrides()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        st = t.stride()
        getattr(s, name)[:] = [st[0], st[1], st[2]]
    if bias is not None:
        st = bias.stride()
        s.bias[:] = [st[0], st[1], st[2]]
    if lse is not None:
        st = lse.stride()
        s.lse[:] = [st[0], st[1]]
    return s


def _expect(t, name, shape, dtype):
    """A caller-supplied tensor must have exactly the shape and dtype the C ABI sizes it
    by (the library derives every extent from q's shape)."""
    if tuple(t.shape) != tuple(shape):
        raise FaError(STATUS["FA_ERR_SHAPE"], f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise FaError(STATUS["FA_ERR_DTYPE"], f"{name} has dtype {t.dtype}, expected {dtype}")


def _same_device(named):
    """Every tensor is device memory of one HIP device (the library dereferences the
    pointers on the GPU)."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise FaError(STATUS["FA_ERR_NULL"], f"{name} is not a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise FaError(STATUS["FA_ERR_NULL"], f"{name} is on {t.device}, expected {dev}")


def _prepare(q, k, v, bias, causal, out, lse, rect=False, check_device=True):
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FaError(STATUS["FA_ERR_SHAPE"], "q, k, v must be 4-D [B, H, N, *]")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dv = v.shape[-1]
    if (not rect and Nk != N) or tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape[:3]) != (B, H, Nk):
        raise FaError(STATUS["FA_ERR_SHAPE"], "q, k, v shapes disagree")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise FaError(STATUS["FA_ERR_DTYPE"], "q, k, v dtypes differ")
    for t in (q, k, v):
        if t.numel() and t.stride(-1) != 1:
            raise FaError(STATUS["FA_ERR_STRIDE"], "innermost axis must be contiguous")
    if bias is not None:
        if bias.dtype != torch.float32:
            raise FaError(STATUS["FA_ERR_DTYPE"], "bias must be float32")
        if bias.dim() == 3:
            bias = bias.unsqueeze(0)
        if bias.dim() != 4 or any(bs not in (1, full) for bs, full in zip(bias.shape, (B, H, N, Nk))) \
                or tuple(bias.shape[2:]) != (N, Nk):
            raise FaError(STATUS["FA_ERR_SHAPE"], f"bias of shape {tuple(bias.shape)} does not "
                          f"broadcast to {(B, H, N, Nk)} as [B|1, H|1, N_q, N_k]")
        bias = bias.expand(B, H, N, Nk)
        if N and Nk and bias.stride(-1) != 1:
            raise FaError(STATUS["FA_ERR_STRIDE"], "bias key axis must be contiguous")
    if out is not None:
        _expect(out, "out", (B, H, N, dv), q.dtype)
    if lse is not None:
        _expect(lse, "lse", (B, H, N), torch.float32)
    if check_device:
        _same_device((("q", q), ("k", k), ("v", v), ("bias", bias), ("out", out), ("lse", lse)))
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    mask = FA_MASK_CAUSAL if causal else FA_MASK_NONE
    strides = make_strides(q, k, v, out, bias, lse)
    if rect:
        return (B, H, N, Nk, d, dv, dt, mask, bias, out, lse, strides)
    return (B, H, N, d, dv, dt, mask, bias, out, lse, strides)


def _workspace_bytes(workspace, like):
    """Size of a caller workspace: a uint8 tensor on the inputs' device, or None."""
    import torch

    if workspace is None:
        return 0
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise FaError(STATUS["FA_ERR_WORKSPACE"], "workspace must be a 1-D uint8 tensor")
    _same_device((("q", like), ("workspace", workspace)))
    return workspace.numel()


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def fa_fwd(q, k, v, bias=None, causal=False, out=None, lse=None, stream=None):
    """Attention forward through fa_fwd. Returns (out, lse).

    q, k: [B, H, N, d]; v: [B, H, N, dv]; bf16 or fp32 (same dtype), on one HIP device.
    bias: None or fp32 broadcastable to [B, H, N, N] (as [B|1, H|1, N, N] or [H, N, N]).
    out / lse are allocated when not given. Enqueued on `stream` (default: torch's
    current stream); no synchronisation.
    """
    B, H, N, d, dv, dt, mask, bias, out, lse, strides = _prepare(q, k, v, bias, causal, out, lse)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), mask, _ptr(out), _ptr(lse),
                      B, H, N, d, dv, ctypes.byref(strides), dt, _stream_handle(stream, q.device))
    _check(st)
    return out, lse


def fa_fwd_qk(q, k, v, bias=None, causal=False, out=None, lse=None, stream=None):
    """Attention forward of N_q query rows against N_k keys through fa_fwd_qk.

    q: [B, H, N_q, d]; k: [B, H, N_k, d]; v: [B, H, N_k, dv]; bias: None or fp32
    broadcastable to [B, H, N_q, N_k]. The causal mask aligns the query rows to the end
    of the keys (key j allowed for row i iff j <= i + N_k - N_q). Returns (out, lse).
    """
    B, H, Nq, Nk, d, dv, dt, mask, bias, out, lse, strides = _prepare(q, k, v, bias, causal, out, lse, rect=True)
    st = lib().fa_fwd_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), mask, _ptr(out), _ptr(lse),
                         B, H, Nq, Nk, d, dv, ctypes.byref(strides), dt, _stream_handle(stream, q.device))
    _check(st)
    return out, lse


def fa_fwd_qk_noalloc(q, k, v, out, lse, bias=None, causal=False, stream=None):
    """fa_fwd_qk through fa_fwd_qk_noalloc, which allocates no device memory: out and lse
    must be given (the binding allocates nothing either). Split problems use the
    library's fixed per-GPU scratch array, so overlapping calls on one GPU race.
    Returns (out, lse)."""
    if out is None or lse is None:
        raise FaError(STATUS["FA_ERR_NULL"], "fa_fwd_qk_noalloc needs out and lse")
    B, H, Nq, Nk, d, dv, dt, mask, bias, out, lse, strides = _prepare(q, k, v, bias, causal, out, lse, rect=True)
    st = lib().fa_fwd_qk_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), mask, _ptr(out), _ptr(lse),
                                 B, H, Nq, Nk, d, dv, ctypes.byref(strides), dt, _stream_handle(stream, q.device))
    _check(st)
    return out, lse


def fa_fwd_qk_workspace_size(B, H, Nq, Nk, d, dv, dtype_code, causal) -> int:
    return int(lib().fa_fwd_qk_workspace_size(B, H, Nq, Nk, d, dv, dtype_code,
                                              FA_MASK_CAUSAL if causal else FA_MASK_NONE))


def fa_fwd_qk_ex(q, k, v, workspace, bias=None, causal=False, out=None, lse=None, stream=None):
    """fa_fwd_qk with a caller-provided workspace (a uint8 device tensor, or None)."""
    B, H, Nq, Nk, d, dv, dt, mask, bias, out, lse, strides = _prepare(q, k, v, bias, causal, out, lse, rect=True)
    nbytes = _workspace_bytes(workspace, q)
    st = lib().fa_fwd_qk_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), mask, _ptr(out), _ptr(lse),
                            B, H, Nq, Nk, d, dv, ctypes.byref(strides), dt,
                            _stream_handle(stream, q.device), _ptr(workspace), nbytes)
    _check(st)
    return out, lse


def fa_fwd_workspace_size(B, H, N, d, dv, dtype_code, causal) -> int:
    return int(lib().fa_fwd_workspace_size(B, H, N, d, dv, dtype_code,
                                           FA_MASK_CAUSAL if causal else FA_MASK_NONE))


def fa_fwd_ex(q, k, v, workspace, bias=None, causal=False, out=None, lse=None, stream=None):
    """fa_fwd with a caller-provided workspace (a uint8 device tensor, or None)."""
    B, H, N, d, dv, dt, mask, bias, out, lse, strides = _prepare(q, k, v, bias, causal, out, lse)
    nbytes = _workspace_bytes(workspace, q)
    st = lib().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), mask, _ptr(out), _ptr(lse),
                         B, H, N, d, dv, ctypes.byref(strides), dt,
                         _stream_handle(stream, q.device), _ptr(workspace), nbytes)
    _check(st)
    return out, lse


def _prepare_bwd(q, k, v, out, lse, grad_out, bias, causal, grad_q, grad_k, grad_v):
    import torch

    if out is None or lse is None or grad_out is None:
        raise FaError(STATUS["FA_ERR_NULL"], "out, lse and grad_out (the forward's O, its "
                      "log-sum-exp and dO) are required")
    B, H, N, d, dv, dt, mask, bias, out, lse, _ = _prepare(q, k, v, bias, causal, out, lse,
                                                           check_device=False)
    _expect(grad_out, "grad_out", (B, H, N, dv), q.dtype)
    for name, t, width in (("grad_q", grad_q, d), ("grad_k", grad_k, d), ("grad_v", grad_v, dv)):
        if t is not None:
            _expect(t, name, (B, H, N, width), q.dtype)
    _same_device((("q", q), ("k", k), ("v", v), ("bias", bias), ("out", out), ("lse", lse),
                  ("grad_out", grad_out), ("grad_q", grad_q), ("grad_k", grad_k), ("grad_v", grad_v)))
    if grad_q is None:
        grad_q = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    if grad_k is None:
        grad_k = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    if grad_v is None:
        grad_v = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    s = FaBwdStrides()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("grad_out", grad_out),
                    ("grad_q", grad_q), ("grad_k", grad_k), ("grad_v", grad_v)):
        if t.numel() and t.stride(-1) != 1:
            raise FaError(STATUS["FA_ERR_STRIDE"], f"{name}: innermost axis must be contiguous")
        st = t.stride()
        getattr(s, name)[:] = [st[0], st[1], st[2]]
    if bias is not None:
        st = bias.stride()
        s.bias[:] = [st[0], st[1], st[2]]
    st = lse.stride()
    s.lse[:] = [st[0], st[1]]
    return B, H, N, d, dv, dt, mask, bias, out, lse, grad_q, grad_k, grad_v, s


def fa_bwd(q, k, v, out, lse, grad_out, bias=None, causal=False, grad_q=None, grad_k=None,
           grad_v=None, stream=None):
    """Gradients through fa_bwd: (grad_q, grad_k, grad_v) of fa_fwd's output for the
    upstream gradient grad_out, from the forward's out and lse. bf16 or fp16 tensors; outputs are
    allocated when not given. Enqueued on `stream` (default: torch's current stream)."""
    (B, H, N, d, dv, dt, mask, bias, out, lse, grad_q, grad_k, grad_v,
     s) = _prepare_bwd(q, k, v, out, lse, grad_out, bias, causal, grad_q, grad_k, grad_v)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(grad_out), _ptr(bias), mask,
                      _ptr(grad_q), _ptr(grad_k), _ptr(grad_v), B, H, N, d, dv, ctypes.byref(s), dt,
                      _stream_handle(stream, q.device))
    _check(st)
    return grad_q, grad_k, grad_v


def fa_bwd_workspace_size(B, H, N, d, dv, dtype_code, causal) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, N, d, dv, dtype_code,
                                           FA_MASK_CAUSAL if causal else FA_MASK_NONE))


def fa_bwd_ex(q, k, v, out, lse, grad_out, workspace, bias=None, causal=False, grad_q=None,
              grad_k=None, grad_v=None, stream=None):
    """fa_bwd with a caller-provided workspace (a uint8 device tensor)."""
    (B, H, N, d, dv, dt, mask, bias, out, lse, grad_q, grad_k, grad_v,
     s) = _prepare_bwd(q, k, v, out, lse, grad_out, bias, causal, grad_q, grad_k, grad_v)
    nbytes = _workspace_bytes(workspace, q)
    st = lib().fa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(grad_out), _ptr(bias),
                         mask, _ptr(grad_q), _ptr(grad_k), _ptr(grad_v), B, H, N, d, dv, ctypes.byref(s),
                         dt, _stream_handle(stream, q.device), _ptr(workspace), nbytes)
    _check(st)
    return grad_q, grad_k, grad_v


def fa_probe_copy(src, dst, stream=None):
    """The streaming copy probe: dst <- src (device tensors of equal byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise FaError(STATUS["FA_ERR_SHAPE"], "src and dst sizes differ")
    _same_device((("src", src), ("dst", dst)))
    _check(lib().fa_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream_handle(stream, src.device)))


def fa_probe_mfma(out, blocks, iters, stream=None):
    """The bf16 matrix-core probe; out: float32 device tensor of blocks * 256 elements.
    Returns the FLOPs the launch performs."""
    import torch

    if out.dtype != torch.float32 or out.numel() < blocks * 256:
        raise FaError(STATUS["FA_ERR_SHAPE"], "out must hold blocks * 256 float32 values")
    _same_device((("out", out),))
    _check(lib().fa_probe_mfma(_ptr(out), int(blocks), int(iters), _stream_handle(stream, out.device)))
    return float(lib().fa_probe_mfma_flops(int(blocks), int(iters)))


def fa_probe_timer_arm(n):
    """Arms kernel-timestamp timing for the calling thread's next n main-kernel launches."""
    if not 0 <= int(n) <= FA_PROBE_TIMER_MAX:
        raise FaError(STATUS["FA_ERR_NULL"], f"n must lie in [0, {FA_PROBE_TIMER_MAX}]")
    _check(lib().fa_probe_timer_arm(int(n)))


def fa_probe_timer_read(n):
    """Waits for the n armed launches and returns their durations in microseconds."""
    buf = (ctypes.c_float * max(int(n), 1))()
    _check(lib().fa_probe_timer_read(buf, int(n)))
    return [float(buf[i]) for i in range(int(n))]


def fa_probe_issue(role, valu_ops, exps, blocks, iters, stream=None):
    """The issue probe (include/fa_probe.h): returns per-wave (shader cycles, 100 MHz
    ticks) of the waves that worked, as two lists, after the launch completes."""
    import torch

    waves = blocks * (4 if role == 0 else 8)
    dev = torch.device("cuda", torch.cuda.current_device())
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(st):  # the zeroed tick buffer is ready on the probe's stream
        out = torch.empty(waves * 64, dtype=torch.float32, device=dev)
        ticks = torch.zeros(2 * waves, dtype=torch.int64, device=dev)
    _check(lib().fa_probe_issue(int(role), int(valu_ops), int(exps), int(blocks), int(iters), _ptr(out),
                                _ptr(ticks), _stream_handle(st, dev)))
    torch.cuda.synchronize(dev)
    t = ticks.view(-1, 2).cpu().tolist()
    return [a for a, b in t if a > 0], [b for a, b in t if a > 0], [w for w, (a, b) in enumerate(t) if a > 0]


def _wave_ticks(ticks, dev):
    import torch

    torch.cuda.synchronize(dev)
    t = ticks.view(-1, 2).cpu().tolist()
    return [a for a, b in t], [b for a, b in t]


def fa_probe_lds(mode, blocks, iters, stream=None):
    """The LDS probe (include/fa_probe.h): per-wave (shader cycles, 100 MHz ticks) lists and
    the launch's duration in ms from events recorded around it on the same stream."""
    import torch

    dev = torch.device("cuda", torch.cuda.current_device())
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(st):  # the zeroed tick buffer is ready on the probe's stream
        out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        ticks = torch.zeros(2 * blocks * 4, dtype=torch.int64, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    _check(lib().fa_probe_lds(int(mode), int(blocks), int(iters), _ptr(out), _ptr(ticks), _stream_handle(st, dev)))
    e1.record(st)
    cyc, rt = _wave_ticks(ticks, dev)
    return cyc, rt, e0.elapsed_time(e1)


def fa_probe_tile(copies, valu_ops, blocks, tiles, src=None, stream=None):
    """The tile-body probe (include/fa_probe.h): per-wave (shader cycles, 100 MHz ticks)
    lists and the launch's duration in ms from events recorded around it on the same stream;
    src: a device tensor of at least 256 KiB when copies = 1."""
    import torch

    dev = torch.device("cuda", torch.cuda.current_device())
    if src is not None:
        _same_device((("src", src),))
        if src.device != dev:
            raise FaError(STATUS["FA_ERR_NULL"], f"src is on {src.device}, expected {dev}")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    nbytes = 0 if src is None else src.numel() * src.element_size()
    with torch.cuda.stream(st):  # the zeroed tick buffer is ready on the probe's stream
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        ticks = torch.zeros(2 * blocks * 4, dtype=torch.int64, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    _check(lib().fa_probe_tile(int(copies), int(valu_ops), int(blocks), int(tiles), _ptr(src), nbytes, _ptr(out),
                               _ptr(ticks), _stream_handle(st, dev)))
    e1.record(st)
    cyc, rt = _wave_ticks(ticks, dev)
    return cyc, rt, e0.elapsed_time(e1)


def fa_probe_read(src, sink, stream=None):
    """The read-only streaming probe over a device tensor; sink: int32 device tensor with
    at least 16 * CU-count elements."""
    import torch

    if sink.dtype != torch.int32:
        raise FaError(STATUS["FA_ERR_SHAPE"], "sink must be int32")
    _same_device((("src", src), ("sink", sink)))
    nbytes = src.numel() * src.element_size()
    _check(lib().fa_probe_read(_ptr(src), nbytes, _ptr(sink), int(sink.numel()), _stream_handle(stream, src.device)))
