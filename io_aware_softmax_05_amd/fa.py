"""Thin ctypes binding over the C ABI in include/fa.h (libfa_gfx950.so).

The functions named like the C entry points (fa_fwd, fa_fwd_f32, fa_bwd,
fa_decode_splitkv, the workspace-size queries, fa_status_string) take the C
parameter list as-is -- device tensors stand in for pointers -- and only
marshal arguments; a non-zero status raises FaError. The lower-case helpers
(forward, backward, decode) additionally check shapes and dtypes and allocate
outputs with torch; every arithmetic step runs in the library's kernels.

torch is used for device memory and streams only. It is imported before the
library is loaded so that both share one HIP runtime. There is no fallback:
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa_gfx950.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "fa.h")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_HIP = -4

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32

# (restype, argtypes) per exported symbol, in header order.
_SIGNATURES = {
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_workspace_size": (_S, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_window": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_tiles": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_bwd_tiles": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_dropout_keep_threshold": (_I, [_F]),
    "fa_fwd_dropout": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _F, _U64, _U32, _P]),
    "fa_bwd_dropout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _I, _F, _I,
                            _F, _U64, _U32, _P]),
    "fa_decode_workspace_size": (_S, [_I, _I, _I, _I]),
    "fa_decode_splitkv": (_I, [_P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_splitkv_window": (_I, [_P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_decode_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
}

FA_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


class LibraryMissing(RuntimeError):
    pass


def header_functions() -> list[str]:
    """Names of the functions include/fa.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fa_[a-z0-9_]+)\s*\(", text, flags=re.M)


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle; raises LibraryMissing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise LibraryMissing(f"{p} is not built; run io_aware_softmax_05_amd.build.build_library()")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().fa_status_string(int(status)).decode()
    except LibraryMissing:
        return f"status {status}"


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)


# ------------------------------------------------------------ C entry points

def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, stream=None) -> None:
    st = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d,
                               float(scale), int(bool(causal)), _stream(stream))
    _check(st, "fa_fwd")


def fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, window, stream=None) -> None:
    st = load_library().fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d,
                                      float(scale), int(window), _stream(stream))
    _check(st, "fa_fwd_window")


def fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, stream=None) -> None:
    st = load_library().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d,
                                   float(scale), int(bool(causal)), _stream(stream))
    _check(st, "fa_fwd_f32")


def fa_fwd_fp8(q, k, vt, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal,
               stream=None) -> None:
    st = load_library().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(vt), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                   _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d, float(scale), int(bool(causal)),
                                   _stream(stream))
    _check(st, "fa_fwd_fp8")


def fa_bwd_workspace_size(B, Hq, Tq, d) -> int:
    return int(load_library().fa_bwd_workspace_size(B, Hq, Tq, d))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, causal,
           stream=None) -> None:
    st = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(workspace), int(ws_bytes), B, Hq, Hkv, Tq, Tk, d, float(scale),
                               int(bool(causal)), _stream(stream))
    _check(st, "fa_bwd")


def fa_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, window,
                  stream=None) -> None:
    st = load_library().fa_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(workspace), int(ws_bytes), B, Hq, Hkv, Tq, Tk, d,
                                      float(scale), int(window), _stream(stream))
    _check(st, "fa_bwd_window")


def fa_fwd_tiles(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, tile_shape, stream=None) -> None:
    st = load_library().fa_fwd_tiles(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d,
                                     float(scale), int(bool(causal)), int(tile_shape), _stream(stream))
    _check(st, "fa_fwd_tiles")


def fa_bwd_tiles(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, causal,
                 tile_shape, stream=None) -> None:
    st = load_library().fa_bwd_tiles(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                     _ptr(dk), _ptr(dv), _ptr(workspace), int(ws_bytes), B, Hq, Hkv, Tq, Tk, d,
                                     float(scale), int(bool(causal)), int(tile_shape), _stream(stream))
    _check(st, "fa_bwd_tiles")


def fa_dropout_keep_threshold(p_drop) -> int:
    """Keep threshold t in [1, 256] for p_drop (raises FaError when unusable)."""
    t = int(load_library().fa_dropout_keep_threshold(float(p_drop)))
    if t < 0:
        raise FaError(t, "fa_dropout_keep_threshold")
    return t


def fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, p_drop, seed, offset,
                   stream=None) -> None:
    st = load_library().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d,
                                       float(scale), int(bool(causal)), float(p_drop), int(seed), int(offset),
                                       _stream(stream))
    _check(st, "fa_fwd_dropout")


def fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, causal,
                   p_drop, seed, offset, stream=None) -> None:
    st = load_library().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(workspace), int(ws_bytes), B, Hq, Hkv, Tq, Tk, d,
                                       float(scale), int(bool(causal)), float(p_drop), int(seed), int(offset),
                                       _stream(stream))
    _check(st, "fa_bwd_dropout")


def fa_decode_workspace_size(B, Hq, Tk_max, d) -> int:
    return int(load_library().fa_decode_workspace_size(B, Hq, Tk_max, d))


def fa_decode_splitkv(q, k_cache, v_cache, seq_lens, o, lse, workspace, ws_bytes, B, Hq, Hkv, Tk_max, d,
                      scale, chunk=0, stream=None) -> None:
    st = load_library().fa_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(o),
                                          _ptr(lse), _ptr(workspace), int(ws_bytes), B, Hq, Hkv, Tk_max, d,
                                          float(scale), int(chunk), _stream(stream))
    _check(st, "fa_decode_splitkv")


def fa_decode_splitkv_window(q, k_cache, v_cache, seq_lens, o, lse, workspace, ws_bytes, B, Hq, Hkv, Tk_max, d,
                             scale, window, chunk=0, stream=None) -> None:
    st = load_library().fa_decode_splitkv_window(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(o),
                                                 _ptr(lse), _ptr(workspace), int(ws_bytes), B, Hq, Hkv, Tk_max,
                                                 d, float(scale), int(window), int(chunk), _stream(stream))
    _check(st, "fa_decode_splitkv_window")


def fa_decode_splitkv_noalloc(q, k_cache, v_cache, seq_lens, o, lse, B, Hq, Hkv, Tk_max, d, scale, chunk=0,
                              stream=None) -> None:
    st = load_library().fa_decode_splitkv_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(o),
                                                  _ptr(lse), B, Hq, Hkv, Tk_max, d, float(scale), int(chunk),
                                                  _stream(stream))
    _check(st, "fa_decode_splitkv_noalloc")


# ------------------------------------------------ tensor-level conveniences
#
# The kernels index every tensor by the sizes passed with q, so a tensor of
# another shape would be read or written past its end. The helpers therefore
# check every tensor's dtype, rank, contiguity and shape against q, and that
# all of them sit on one GPU, before anything reaches the library.

def _need(t, dtype, ndim: int, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
        got = f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}" if isinstance(t, torch.Tensor) else type(t)
        raise ValueError(f"{name} must be a contiguous {dtype} tensor with {ndim} dims, got {got}")


def _need_shape(t: torch.Tensor, shape, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _one_gpu(**tensors) -> torch.device:
    devs = {t.device for t in tensors.values() if t is not None}
    if len(devs) != 1:
        raise ValueError("all tensors must be on one device, got " +
                         ", ".join(f"{n}: {t.device}" for n, t in tensors.items() if t is not None))
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {dev}")
    return dev


def _check_forward_args(q, k, v) -> None:
    dt = q.dtype if isinstance(q, torch.Tensor) else None
    if dt not in (torch.bfloat16, torch.float32):
        raise ValueError(f"q must be bfloat16 or float32, got {dt}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, dt, 4, name)
    B, Hq, _, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    _need_shape(k, (B, Hkv, Tk, d), "k")
    _need_shape(v, k.shape, "v")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError(f"the number of query heads ({Hq}) must be a multiple of the KV heads ({Hkv})")
    _one_gpu(q=q, k=k, v=v)


def _check_backward_args(q, k, v, o, dout, lse) -> None:
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, torch.bfloat16, 4, name)
    _need(lse, torch.float32, 3, "lse")
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    _need_shape(k, (B, Hkv, Tk, d), "k")
    _need_shape(v, k.shape, "v")
    _need_shape(o, q.shape, "o")
    _need_shape(dout, q.shape, "dout")
    _need_shape(lse, (B, Hq, Tq), "lse")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError(f"the number of query heads ({Hq}) must be a multiple of the KV heads ({Hkv})")
    _one_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse)


def _check_decode_args(q, k_cache, v_cache, seq_lens, workspace=None, ws_bytes: int = 0) -> None:
    _need(q, torch.bfloat16, 3, "q")
    _need(k_cache, torch.bfloat16, 4, "k_cache")
    _need(v_cache, torch.bfloat16, 4, "v_cache")
    _need(seq_lens, torch.int32, 1, "seq_lens")
    B, Hq, d = q.shape
    Hkv, Tk_max = k_cache.shape[1], k_cache.shape[2]
    _need_shape(k_cache, (B, Hkv, Tk_max, d), "k_cache")
    _need_shape(v_cache, k_cache.shape, "v_cache")
    _need_shape(seq_lens, (B,), "seq_lens")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError(f"the number of query heads ({Hq}) must be a multiple of the KV heads ({Hkv})")
    if workspace is not None:
        _need(workspace, torch.uint8, 1, "workspace")
        if workspace.numel() < ws_bytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {ws_bytes} are needed")
    _one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, workspace=workspace)


def forward(q, k, v, causal: bool = False, scale: float | None = None, with_lse: bool = True, stream=None):
    """O (and LSE) for q [B,Hq,Tq,d], k and v [B,Hkv,Tk,d]; bf16 or fp32."""
    _check_forward_args(q, k, v)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    scale = d ** -0.5 if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if with_lse else None
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    fn(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, causal, stream)
    return o, lse


def backward(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, stream=None):
    """dQ, dK, dV (bf16) by recomputation from the saved LSE."""
    _check_backward_args(q, k, v, o, dout, lse)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    scale = d ** -0.5 if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa_bwd_workspace_size(B, Hq, Tq, d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, Tq, Tk, d, scale, causal, stream)
    return dq, dk, dv


def decode(q, k_cache, v_cache, seq_lens, scale: float | None = None, chunk: int = 0, workspace=None,
           stream=None):
    """O [B,Hq,d] and LSE [B,Hq] for one query token per head."""
    _check_decode_args(q, k_cache, v_cache, seq_lens)
    B, Hq, d = q.shape
    Hkv, Tk_max = k_cache.shape[1], k_cache.shape[2]
    scale = d ** -0.5 if scale is None else scale
    ws_bytes = fa_decode_workspace_size(B, Hq, Tk_max, d)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check_decode_args(q, k_cache, v_cache, seq_lens, workspace, ws_bytes)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    fa_decode_splitkv(q, k_cache, v_cache, seq_lens, o, lse, workspace, workspace.numel(), B, Hq, Hkv, Tk_max, d,
                      scale, chunk, stream)
    return o, lse
