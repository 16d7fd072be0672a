"""Thin Python binding of ``libboost_lrblock.so`` (argument marshalling only).

Every step of the block runs in the HIP library. PyTorch is used for device
memory and streams: tensors are passed as raw device pointers together with
``torch.cuda.current_stream()``. The binding fails loudly when the library is
missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libboost_lrblock.so")

ABI_VERSION = 1
DT_F32, DT_BF16 = 0, 1
ACT_IDENTITY, ACT_SILU = 0, 1
_ACTS = {"identity": ACT_IDENTITY, "svd": ACT_IDENTITY, "silu": ACT_SILU, "cola": ACT_SILU}
_DTYPES = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}


class BoostError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str, fn: str):
        super().__init__(f"{fn}: {name} ({status}): {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class LrblockDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("norm", ctypes.c_int32), ("T", ctypes.c_int64), ("d", ctypes.c_int64),
                ("r", ctypes.c_int64), ("G", ctypes.c_int64), ("d_out", ctypes.c_int64),
                ("d_norm", ctypes.c_int64), ("eps", ctypes.c_float)]


class LrmlpDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("T", ctypes.c_int64), ("d", ctypes.c_int64),
                ("r", ctypes.c_int64), ("ffn", ctypes.c_int64), ("eps", ctypes.c_float)]


class BtpShareDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32), ("T", ctypes.c_int64),
                ("r", ctypes.c_int64), ("d_shard", ctypes.c_int64)]


_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SIGS = {
    "boost_abi_version": ([], ctypes.c_int),
    "boost_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "boost_last_error_detail": ([], ctypes.c_char_p),
    "boost_lrblock_workspace_size": ([ctypes.POINTER(LrblockDesc), ctypes.c_int, ctypes.POINTER(_SZ)], ctypes.c_int),
    "boost_lrblock_fwd": ([ctypes.POINTER(LrblockDesc)] + [_VP] * 7 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_lrblock_bwd": ([ctypes.POINTER(LrblockDesc)] + [_VP] * 11 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_lrblock_fwd_noalloc": ([ctypes.POINTER(LrblockDesc)] + [_VP] * 7 + [_VP], ctypes.c_int),
    "boost_lrmlp_workspace_size": ([ctypes.POINTER(LrmlpDesc), ctypes.c_int, ctypes.POINTER(_SZ)], ctypes.c_int),
    "boost_lrmlp_fwd": ([ctypes.POINTER(LrmlpDesc)] + [_VP] * 10 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_lrmlp_bwd": ([ctypes.POINTER(LrmlpDesc)] + [_VP] * 16 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_lrblock_fwd_chained": ([ctypes.POINTER(LrblockDesc)] + [_VP] * 10 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_lrblock_bwd_chained": ([ctypes.POINTER(LrblockDesc)] + [_VP] * 12 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_lrmlp_fwd_chained": ([ctypes.POINTER(LrmlpDesc)] + [_VP] * 13 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_lrmlp_bwd_chained": ([ctypes.POINTER(LrmlpDesc)] + [_VP] * 17 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_attn_standin_fwd": ([ctypes.c_int, ctypes.c_int64, ctypes.c_int64, _VP, _VP, _VP], ctypes.c_int),
    "boost_attn_standin_bwd": ([ctypes.c_int, ctypes.c_int64, ctypes.c_int64, _VP, _VP, _VP], ctypes.c_int),
    "boost_btp_share_workspace_size": ([ctypes.POINTER(BtpShareDesc), ctypes.c_int, ctypes.POINTER(_SZ)],
                                       ctypes.c_int),
    "boost_btp_share_fwd": ([ctypes.POINTER(BtpShareDesc)] + [_VP] * 6 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_btp_share_bwd": ([ctypes.POINTER(BtpShareDesc)] + [_VP] * 10 + [_VP, _SZ, _VP], ctypes.c_int),
    "boost_profiler_enable": ([ctypes.c_char_p, ctypes.c_int], ctypes.c_int),
    "boost_profiler_report": ([ctypes.c_char_p, _SZ], ctypes.c_int),
    "boost_profiler_disable": ([], ctypes.c_int),
    "boost_profiler_serialize": ([ctypes.c_int], ctypes.c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m rank_bottleneck_online_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        if L.boost_abi_version() != ABI_VERSION:
            raise RuntimeError("libboost_lrblock.so ABI version mismatch")
        _lib = L
    return _lib


def _check(status: int, fn: str) -> None:
    if status != 0:
        L = lib()
        raise BoostError(status, L.boost_status_string(status).decode(), L.boost_last_error_detail().decode(), fn)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _arg(t, shape, dtype, like, name):
    """Check an operand against the shape and dtype the descriptor implies
    (the C ABI takes plain pointers and cannot)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, shape, dtype, like, name):
    return None if t is None else _arg(t, shape, dtype, like, name)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _anchor(x, name):
    """The tensor every other operand is checked against: on the GPU,
    contiguous, bf16 or fp32."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(x).__name__}")
    if not x.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    _dtype_code(x)
    return _arg(x, x.shape, x.dtype, x, name)


F32 = torch.float32


def _block_args(x, g, A_cat, B, norm):
    T, d = x.shape
    G, r, d_out = B.shape
    if norm:
        _arg(g, (d,), x.dtype, x, "g")
    _arg(A_cat, (d, G * r), x.dtype, x, "A_cat")
    _arg(B, (G, r, d_out), x.dtype, x, "B")


def _block_saved(x, H, sumsq, dY, G, r, d_out, norm):
    T = x.shape[0]
    _arg(H, (T, G * r), F32, x, "H")
    if norm:
        _arg(sumsq, (T,), F32, x, "sumsq")
    _arg(dY, (G, T, d_out), x.dtype, x, "dY")


def _block_grads(x, dx, dg, dA, dB, G, r, d_out, norm):
    T, d = x.shape
    _arg(dx, (T, d), x.dtype, x, "dx")
    if norm:
        _arg(dg, (d,), F32, x, "dg")
    _arg(dA, (d, G * r), F32, x, "dA_cat")
    _arg(dB, (G, r, d_out), F32, x, "dB")


def _mlp_args(x, g, A1_cat, B1, A2, B2):
    T, d = x.shape
    _, r, ffn = B1.shape
    _arg(g, (d,), x.dtype, x, "g")
    _arg(A1_cat, (d, 2 * r), x.dtype, x, "A1_cat")
    _arg(B1, (2, r, ffn), x.dtype, x, "B1")
    _arg(A2, (ffn, r), x.dtype, x, "A2")
    _arg(B2, (r, d), x.dtype, x, "B2")


def _mlp_saved(x, H1, H2, sumsq, dY, r):
    T, d = x.shape
    _arg(H1, (T, 2 * r), F32, x, "H1")
    _arg(H2, (T, r), F32, x, "H2")
    _arg(sumsq, (T,), F32, x, "sumsq")
    _arg(dY, (T, d), x.dtype, x, "dY")


def _mlp_grads(x, dx, dg, dA1, dB1, dA2, dB2, r, ffn):
    T, d = x.shape
    _arg(dx, (T, d), x.dtype, x, "dx")
    _arg(dg, (d,), F32, x, "dg")
    _arg(dA1, (d, 2 * r), F32, x, "dA1_cat")
    _arg(dB1, (2, r, ffn), F32, x, "dB1")
    _arg(dA2, (ffn, r), F32, x, "dA2")
    _arg(dB2, (r, d), F32, x, "dB2")


def _mlp_fwd_outs(x, Y, H1, H2, sumsq, r):
    T, d = x.shape
    _arg(Y, (T, d), x.dtype, x, "Y")
    _arg(H1, (T, 2 * r), F32, x, "H1")
    _arg(H2, (T, r), F32, x, "H2")
    _opt(sumsq, (T,), F32, x, "sumsq")


def _btp_args(z, B_s, g_s, A_s):
    T, r = z.shape
    ds = B_s.shape[1]
    _arg(B_s, (r, ds), z.dtype, z, "B_s")
    _arg(g_s, (ds,), z.dtype, z, "g_s")
    _arg(A_s, (ds, r), z.dtype, z, "A_s")


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _act(act) -> int:
    if isinstance(act, int):
        return act
    return _ACTS[act]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")
    return _DTYPES[t.dtype]


def _ws(nbytes: int, device, ws):
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        if ws.device != device:
            raise ValueError(f"workspace is on {ws.device}, expected {device}")
        if _nbytes(ws) < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def upload(a, dtype: str, device="cuda") -> torch.Tensor:
    """Copy an fp64 array of dtype-representable values ("bf16" or "f32") to
    a device tensor of that dtype, bit-exactly."""
    import numpy as np

    from . import synth
    bits = synth.storage_bits(np.ascontiguousarray(a), dtype)
    if dtype == "bf16":
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(bits)
    return t.to(device)


def _f32(shape, device):
    return torch.empty(shape, dtype=torch.float32, device=device)


# ---------------------------------------------------------------------------
# Grouped block
# ---------------------------------------------------------------------------

def lrblock_desc(T, d, r, G, d_out, dtype, act="silu", norm=True, eps=1e-5, d_norm=None) -> LrblockDesc:
    return LrblockDesc(ABI_VERSION, dtype, _act(act), int(bool(norm)), T, d, r, G, d_out,
                       d if d_norm is None else d_norm, eps)


def lrblock_workspace_size(desc: LrblockDesc, is_bwd: bool) -> int:
    n = _SZ(0)
    _check(lib().boost_lrblock_workspace_size(ctypes.byref(desc), int(is_bwd), ctypes.byref(n)),
           "boost_lrblock_workspace_size")
    return n.value


def lrblock_fwd(x, g, A_cat, B, act="silu", norm=True, eps=1e-5, d_norm=None, out=None, ws=None, stream=None):
    """Returns (Y[G,T,d_out], H[T,G*r] fp32, sumsq[T] fp32 or None)."""
    _anchor(x, "x")
    T, d = x.shape
    G, r, d_out = B.shape
    _block_args(x, g, A_cat, B, norm)
    desc = lrblock_desc(T, d, r, G, d_out, _dtype_code(x), act, norm, eps, d_norm)
    if out is None:
        out = (torch.empty((G, T, d_out), dtype=x.dtype, device=x.device), _f32((T, G * r), x.device),
               _f32((T,), x.device) if norm else None)
    Y, H, sumsq = out
    _arg(Y, (G, T, d_out), x.dtype, x, "Y")
    _arg(H, (T, G * r), F32, x, "H")
    if norm:
        _arg(sumsq, (T,), F32, x, "sumsq")
    ws = _ws(lrblock_workspace_size(desc, False), x.device, ws)
    _check(lib().boost_lrblock_fwd(ctypes.byref(desc), _ptr(x), _ptr(g) if norm else None, _ptr(A_cat), _ptr(B),
                                   _ptr(Y), _ptr(H), _ptr(sumsq), _ptr(ws), _nbytes(ws), _stream(stream)),
           "boost_lrblock_fwd")
    return Y, H, sumsq


def lrblock_fwd_noalloc(x, g, A_cat, B, act="silu", norm=True, eps=1e-5, d_norm=None, out=None, stream=None):
    """The forward with the library's fixed scratch instead of a workspace;
    `out` = (Y, H, sumsq) must be given (nothing is allocated here)."""
    _anchor(x, "x")
    T, d = x.shape
    G, r, d_out = B.shape
    _block_args(x, g, A_cat, B, norm)
    desc = lrblock_desc(T, d, r, G, d_out, _dtype_code(x), act, norm, eps, d_norm)
    if out is None:
        raise ValueError("lrblock_fwd_noalloc needs preallocated outputs (Y, H, sumsq)")
    Y, H, sumsq = out
    _arg(Y, (G, T, d_out), x.dtype, x, "Y")
    _arg(H, (T, G * r), F32, x, "H")
    if norm:
        _arg(sumsq, (T,), F32, x, "sumsq")
    _check(lib().boost_lrblock_fwd_noalloc(ctypes.byref(desc), _ptr(x), _ptr(g) if norm else None, _ptr(A_cat),
                                           _ptr(B), _ptr(Y), _ptr(H), _ptr(sumsq), _stream(stream)),
           "boost_lrblock_fwd_noalloc")
    return Y, H, sumsq


def lrblock_bwd(x, g, A_cat, B, H, sumsq, dY, act="silu", norm=True, eps=1e-5, d_norm=None, out=None, ws=None,
                stream=None):
    """Returns (dx[T,d], dg[d] fp32 or None, dA_cat fp32, dB fp32)."""
    _anchor(x, "x")
    T, d = x.shape
    G, r, d_out = B.shape
    _block_args(x, g, A_cat, B, norm)
    _block_saved(x, H, sumsq, dY, G, r, d_out, norm)
    desc = lrblock_desc(T, d, r, G, d_out, _dtype_code(x), act, norm, eps, d_norm)
    if out is None:
        out = (torch.empty_like(x), _f32((d,), x.device) if norm else None, _f32((d, G * r), x.device),
               _f32((G, r, d_out), x.device))
    dx, dg, dA, dB = out
    _block_grads(x, dx, dg, dA, dB, G, r, d_out, norm)
    ws = _ws(lrblock_workspace_size(desc, True), x.device, ws)
    _check(lib().boost_lrblock_bwd(ctypes.byref(desc), _ptr(x), _ptr(g) if norm else None, _ptr(A_cat), _ptr(B),
                                   _ptr(H), _ptr(sumsq) if norm else None, _ptr(dY), _ptr(dx), _ptr(dg),
                                   _ptr(dA), _ptr(dB), _ptr(ws), _nbytes(ws), _stream(stream)),
           "boost_lrblock_bwd")
    return dx, dg, dA, dB


def lrblock_fwd_chained(x, g, A_cat, B, residual=None, sumsq_in=None, sumsq_next=False, act="silu", norm=True,
                        eps=1e-5, d_norm=None, out=None, ws=None, stream=None):
    """Forward inside a layer: Y = residual + S @ B (G = 1) when residual is
    given, the statistic of x taken from sumsq_in when given, and the next
    block's statistic sumsq_next[T] when asked. Returns (Y, H, sumsq or
    None, sumsq_next or None)."""
    _anchor(x, "x")
    T, d = x.shape
    G, r, d_out = B.shape
    _block_args(x, g, A_cat, B, norm)
    _opt(residual, (T, d_out), x.dtype, x, "residual")
    _opt(sumsq_in, (T,), F32, x, "sumsq_in")
    desc = lrblock_desc(T, d, r, G, d_out, _dtype_code(x), act, norm, eps, d_norm)
    if out is None:
        out = (torch.empty((G, T, d_out), dtype=x.dtype, device=x.device), _f32((T, G * r), x.device),
               _f32((T,), x.device) if norm and sumsq_in is None else None,
               _f32((T,), x.device) if sumsq_next else None)
    Y, H, sumsq, snext = out
    _arg(Y, (G, T, d_out), x.dtype, x, "Y")
    _arg(H, (T, G * r), F32, x, "H")
    _opt(sumsq, (T,), F32, x, "sumsq")
    _opt(snext, (T,), F32, x, "sumsq_next")
    ws = _ws(lrblock_workspace_size(desc, False), x.device, ws)
    _check(lib().boost_lrblock_fwd_chained(ctypes.byref(desc), _ptr(x), _ptr(g) if norm else None, _ptr(A_cat),
                                           _ptr(B), _ptr(residual), _ptr(sumsq_in), _ptr(Y), _ptr(H), _ptr(sumsq),
                                           _ptr(snext), _ptr(ws), _nbytes(ws), _stream(stream)),
           "boost_lrblock_fwd_chained")
    return Y, H, sumsq, snext


def lrblock_bwd_chained(x, g, A_cat, B, H, sumsq, dY, dx_add=None, act="silu", norm=True, eps=1e-5, d_norm=None,
                        out=None, ws=None, stream=None):
    """Backward inside a layer: dx also receives dx_add (the residual path).
    Returns (dx, dg or None, dA_cat, dB)."""
    _anchor(x, "x")
    T, d = x.shape
    G, r, d_out = B.shape
    _block_args(x, g, A_cat, B, norm)
    _block_saved(x, H, sumsq, dY, G, r, d_out, norm)
    _opt(dx_add, (T, d), x.dtype, x, "dx_add")
    desc = lrblock_desc(T, d, r, G, d_out, _dtype_code(x), act, norm, eps, d_norm)
    if out is None:
        out = (torch.empty_like(x), _f32((d,), x.device) if norm else None, _f32((d, G * r), x.device),
               _f32((G, r, d_out), x.device))
    dx, dg, dA, dB = out
    _block_grads(x, dx, dg, dA, dB, G, r, d_out, norm)
    ws = _ws(lrblock_workspace_size(desc, True), x.device, ws)
    _check(lib().boost_lrblock_bwd_chained(ctypes.byref(desc), _ptr(x), _ptr(g) if norm else None, _ptr(A_cat),
                                           _ptr(B), _ptr(H), _ptr(sumsq) if norm else None, _ptr(dY),
                                           _ptr(dx_add), _ptr(dx), _ptr(dg), _ptr(dA), _ptr(dB), _ptr(ws),
                                           _nbytes(ws), _stream(stream)),
           "boost_lrblock_bwd_chained")
    return dx, dg, dA, dB


def attn_standin_fwd(qkv, out=None, stream=None):
    """a = q + k + v for qkv[3,T,d]."""
    _anchor(qkv, "qkv")
    _, T, d = qkv.shape
    if qkv.shape[0] != 3:
        raise ValueError(f"qkv has shape {tuple(qkv.shape)}, expected (3, T, d)")
    a = out if out is not None else torch.empty((T, d), dtype=qkv.dtype, device=qkv.device)
    _arg(a, (T, d), qkv.dtype, qkv, "a")
    _check(lib().boost_attn_standin_fwd(_dtype_code(qkv), T, d, _ptr(qkv), _ptr(a), _stream(stream)),
           "boost_attn_standin_fwd")
    return a


def attn_standin_bwd(da, out=None, stream=None):
    """dqkv[3,T,d] = (da, da, da)."""
    _anchor(da, "da")
    T, d = da.shape
    dqkv = out if out is not None else torch.empty((3, T, d), dtype=da.dtype, device=da.device)
    _arg(dqkv, (3, T, d), da.dtype, da, "dqkv")
    _check(lib().boost_attn_standin_bwd(_dtype_code(da), T, d, _ptr(da), _ptr(dqkv), _stream(stream)),
           "boost_attn_standin_bwd")
    return dqkv


# ---------------------------------------------------------------------------
# MLP
# ---------------------------------------------------------------------------

def lrmlp_desc(T, d, r, ffn, dtype, act="silu", eps=1e-5) -> LrmlpDesc:
    return LrmlpDesc(ABI_VERSION, dtype, _act(act), 0, T, d, r, ffn, eps)


def lrmlp_workspace_size(desc: LrmlpDesc, is_bwd: bool) -> int:
    n = _SZ(0)
    _check(lib().boost_lrmlp_workspace_size(ctypes.byref(desc), int(is_bwd), ctypes.byref(n)),
           "boost_lrmlp_workspace_size")
    return n.value


def lrmlp_fwd(x, g, A1_cat, B1, A2, B2, act="silu", eps=1e-5, out=None, ws=None, stream=None):
    """Returns (Y[T,d], H1[T,2r] fp32, H2[T,r] fp32, sumsq[T] fp32)."""
    _anchor(x, "x")
    T, d = x.shape
    r, ffn = B1.shape[1], B1.shape[2]
    _mlp_args(x, g, A1_cat, B1, A2, B2)
    desc = lrmlp_desc(T, d, r, ffn, _dtype_code(x), act, eps)
    if out is None:
        out = (torch.empty_like(x), _f32((T, 2 * r), x.device), _f32((T, r), x.device), _f32((T,), x.device))
    Y, H1, H2, sumsq = out
    _mlp_fwd_outs(x, Y, H1, H2, sumsq, r)
    ws = _ws(lrmlp_workspace_size(desc, False), x.device, ws)
    _check(lib().boost_lrmlp_fwd(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(A1_cat), _ptr(B1), _ptr(A2), _ptr(B2),
                                 _ptr(Y), _ptr(H1), _ptr(H2), _ptr(sumsq), _ptr(ws), _nbytes(ws), _stream(stream)),
           "boost_lrmlp_fwd")
    return Y, H1, H2, sumsq


def lrmlp_bwd(x, g, A1_cat, B1, A2, B2, H1, H2, sumsq, dY, act="silu", eps=1e-5, out=None, ws=None, stream=None):
    """Returns (dx, dg, dA1_cat, dB1, dA2, dB2); all gradients but dx are fp32."""
    _anchor(x, "x")
    T, d = x.shape
    r, ffn = B1.shape[1], B1.shape[2]
    _mlp_args(x, g, A1_cat, B1, A2, B2)
    desc = lrmlp_desc(T, d, r, ffn, _dtype_code(x), act, eps)
    if out is None:
        dev = x.device
        out = (torch.empty_like(x), _f32((d,), dev), _f32((d, 2 * r), dev), _f32((2, r, ffn), dev),
               _f32((ffn, r), dev), _f32((r, d), dev))
    dx, dg, dA1, dB1, dA2, dB2 = out
    _mlp_saved(x, H1, H2, sumsq, dY, r)
    _mlp_grads(x, dx, dg, dA1, dB1, dA2, dB2, r, ffn)
    ws = _ws(lrmlp_workspace_size(desc, True), x.device, ws)
    _check(lib().boost_lrmlp_bwd(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(A1_cat), _ptr(B1), _ptr(A2), _ptr(B2),
                                 _ptr(H1), _ptr(H2), _ptr(sumsq), _ptr(dY), _ptr(dx), _ptr(dg), _ptr(dA1),
                                 _ptr(dB1), _ptr(dA2), _ptr(dB2), _ptr(ws), _nbytes(ws), _stream(stream)),
           "boost_lrmlp_bwd")
    return dx, dg, dA1, dB1, dA2, dB2


def lrmlp_fwd_chained(x, g, A1_cat, B1, A2, B2, residual=None, sumsq_in=None, sumsq_next=False, act="silu",
                      eps=1e-5, out=None, ws=None, stream=None):
    """Forward inside a layer (see :func:`lrblock_fwd_chained`). Returns (Y,
    H1, H2, sumsq or None, sumsq_next or None)."""
    _anchor(x, "x")
    T, d = x.shape
    r, ffn = B1.shape[1], B1.shape[2]
    _mlp_args(x, g, A1_cat, B1, A2, B2)
    desc = lrmlp_desc(T, d, r, ffn, _dtype_code(x), act, eps)
    if out is None:
        dev = x.device
        out = (torch.empty_like(x), _f32((T, 2 * r), dev), _f32((T, r), dev),
               _f32((T,), dev) if sumsq_in is None else None, _f32((T,), dev) if sumsq_next else None)
    Y, H1, H2, sumsq, snext = out
    _opt(residual, (T, d), x.dtype, x, "residual")
    _opt(sumsq_in, (T,), F32, x, "sumsq_in")
    _mlp_fwd_outs(x, Y, H1, H2, sumsq, r)
    _opt(snext, (T,), F32, x, "sumsq_next")
    ws = _ws(lrmlp_workspace_size(desc, False), x.device, ws)
    _check(lib().boost_lrmlp_fwd_chained(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(A1_cat), _ptr(B1), _ptr(A2),
                                         _ptr(B2), _ptr(residual), _ptr(sumsq_in), _ptr(Y), _ptr(H1), _ptr(H2),
                                         _ptr(sumsq), _ptr(snext), _ptr(ws), _nbytes(ws), _stream(stream)),
           "boost_lrmlp_fwd_chained")
    return Y, H1, H2, sumsq, snext


def lrmlp_bwd_chained(x, g, A1_cat, B1, A2, B2, H1, H2, sumsq, dY, dx_add=None, act="silu", eps=1e-5, out=None,
                      ws=None, stream=None):
    """Backward inside a layer: dx also receives dx_add. Returns (dx, dg,
    dA1_cat, dB1, dA2, dB2)."""
    _anchor(x, "x")
    T, d = x.shape
    r, ffn = B1.shape[1], B1.shape[2]
    _mlp_args(x, g, A1_cat, B1, A2, B2)
    desc = lrmlp_desc(T, d, r, ffn, _dtype_code(x), act, eps)
    if out is None:
        dev = x.device
        out = (torch.empty_like(x), _f32((d,), dev), _f32((d, 2 * r), dev), _f32((2, r, ffn), dev),
               _f32((ffn, r), dev), _f32((r, d), dev))
    dx, dg, dA1, dB1, dA2, dB2 = out
    _mlp_saved(x, H1, H2, sumsq, dY, r)
    _mlp_grads(x, dx, dg, dA1, dB1, dA2, dB2, r, ffn)
    _opt(dx_add, (T, d), x.dtype, x, "dx_add")
    ws = _ws(lrmlp_workspace_size(desc, True), x.device, ws)
    _check(lib().boost_lrmlp_bwd_chained(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(A1_cat), _ptr(B1), _ptr(A2),
                                         _ptr(B2), _ptr(H1), _ptr(H2), _ptr(sumsq), _ptr(dY), _ptr(dx_add),
                                         _ptr(dx), _ptr(dg), _ptr(dA1), _ptr(dB1), _ptr(dA2), _ptr(dB2), _ptr(ws),
                                         _nbytes(ws), _stream(stream)),
           "boost_lrmlp_bwd_chained")
    return dx, dg, dA1, dB1, dA2, dB2


# ---------------------------------------------------------------------------
# Tensor-parallel share
# ---------------------------------------------------------------------------

def btp_desc(T, r, d_shard, dtype) -> BtpShareDesc:
    return BtpShareDesc(ABI_VERSION, dtype, T, r, d_shard)


def btp_workspace_size(desc: BtpShareDesc, is_bwd: bool) -> int:
    n = _SZ(0)
    _check(lib().boost_btp_share_workspace_size(ctypes.byref(desc), int(is_bwd), ctypes.byref(n)),
           "boost_btp_share_workspace_size")
    return n.value


def btp_share_fwd(z, B_s, g_s, A_s, out=None, ws=None, stream=None):
    """Returns (p[T,r], s[T] fp32)."""
    _anchor(z, "z")
    T, r = z.shape
    ds = B_s.shape[1]
    _btp_args(z, B_s, g_s, A_s)
    desc = btp_desc(T, r, ds, _dtype_code(z))
    if out is None:
        out = (torch.empty_like(z), _f32((T,), z.device))
    p, s = out
    _arg(p, (T, r), z.dtype, z, "p")
    _arg(s, (T,), F32, z, "s")
    ws = _ws(btp_workspace_size(desc, False), z.device, ws)
    _check(lib().boost_btp_share_fwd(ctypes.byref(desc), _ptr(z), _ptr(B_s), _ptr(g_s), _ptr(A_s), _ptr(p), _ptr(s),
                                     _ptr(ws), _nbytes(ws), _stream(stream)), "boost_btp_share_fwd")
    return p, s


def btp_share_bwd(z, B_s, g_s, A_s, dp, ds_, out=None, ws=None, stream=None):
    """Returns (dz[T,r], dB_s, dg_s, dA_s) with the weight/gain gradients fp32."""
    _anchor(z, "z")
    T, r = z.shape
    dsh = B_s.shape[1]
    _btp_args(z, B_s, g_s, A_s)
    _arg(dp, (T, r), z.dtype, z, "dp")
    _arg(ds_, (T,), F32, z, "ds")
    desc = btp_desc(T, r, dsh, _dtype_code(z))
    if out is None:
        dev = z.device
        out = (torch.empty_like(z), _f32((r, dsh), dev), _f32((dsh,), dev), _f32((dsh, r), dev))
    dz, dB, dg, dA = out
    _arg(dz, (T, r), z.dtype, z, "dz")
    _arg(dB, (r, dsh), F32, z, "dB_s")
    _arg(dg, (dsh,), F32, z, "dg_s")
    _arg(dA, (dsh, r), F32, z, "dA_s")
    ws = _ws(btp_workspace_size(desc, True), z.device, ws)
    _check(lib().boost_btp_share_bwd(ctypes.byref(desc), _ptr(z), _ptr(B_s), _ptr(g_s), _ptr(A_s), _ptr(dp),
                                     _ptr(ds_), _ptr(dz), _ptr(dB), _ptr(dg), _ptr(dA), _ptr(ws), _nbytes(ws),
                                     _stream(stream)), "boost_btp_share_bwd")
    return dz, dB, dg, dA


# ---------------------------------------------------------------------------
# Kernel timing
# ---------------------------------------------------------------------------

def profiler_enable(name_filter: str | None = None, max_records: int = 4096) -> None:
    _check(lib().boost_profiler_enable(name_filter.encode() if name_filter else None, max_records),
           "boost_profiler_enable")


def profiler_report() -> dict:
    """{label: (count, total_ms)} of the launches timed since the last report."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(lib().boost_profiler_report(buf, len(buf)), "boost_profiler_report")
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def profiler_disable() -> None:
    _check(lib().boost_profiler_disable(), "boost_profiler_disable")


def profiler_serialize(on: bool) -> None:
    """Weight gradients on the caller's stream (True) or the side stream."""
    _check(lib().boost_profiler_serialize(1 if on else 0), "boost_profiler_serialize")
