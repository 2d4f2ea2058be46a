"""Python binding of libattn (fused softmax attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/attn.h.  PyTorch supplies device memory
and the current stream.  There is no fallback path: if libattn.so is missing
or a call is rejected, an exception is raised.

    o, lse = fwd(q, k, v, scale=..., mode="dot"|"rbf", gamma=..., causal=...,
                 window=..., n_reg=..., sink=...)
    o, lse = decode(q, k, v, ..., num_splits=0)
    stream_append(k_new, v_new, k_cache, v_cache, n_sink=4, window=W, pos=p)
    o, lse = stream_decode(q, k_cache, v_cache, n_sink=4, window=W, pos=p, ...)

q (N, Hq, L, E), k and v (N, Hkv, S, E), all bf16 or all float32 (bwd: bf16),
contiguous, on one GPU; sink (Hq,) float32.  Returns o like q and lse
(N, Hq, L) float32.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_DTYPE",
          -4: "ATTN_ERR_UNSUPPORTED", -5: "ATTN_ERR_ALIGN", -6: "ATTN_ERR_WORKSPACE",
          -7: "ATTN_ERR_HIP", -8: "ATTN_ERR_ARG"}
BF16, F32 = 0, 1
MODES = {"dot": 0, "rbf": 1}

EXPORTS = ("attn_fwd", "attn_fwd_biased", "attn_bwd", "attn_bwd_workspace_bytes", "attn_decode", "attn_decode_num_splits", "attn_decode_workspace_bytes",
           "attn_decode_noalloc",
           "attn_stream_append", "attn_stream_decode", "attn_stream_decode_workspace_bytes",
           "attn_socket_hash", "attn_socket_code_bytes", "attn_socket_decode", "attn_socket_decode_workspace_bytes",
           "attn_status_string", "attn_last_error",
           "attn_probe_sink_words", "attn_probe_read", "attn_probe_copy")


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libattn.so (built in-tree by softmax_attention_attn_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m softmax_attention_attn_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        I, F, P, Z = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        lib.attn_fwd.restype = I
        lib.attn_fwd.argtypes = [I, I, I, I, I, I, I, P, P, P, I, F, F, I, I, I, P, P, P, P]
        LLb = ctypes.c_longlong
        lib.attn_fwd_biased.restype = I
        lib.attn_fwd_biased.argtypes = [I, I, I, I, I, I, I, P, P, P, I, F, F, I, I, I, P, I, P, LLb, LLb, P, P, P, P]
        lib.attn_bwd.restype = I
        lib.attn_bwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, I, F, F, I, I, I, P, P, P, P, P, P, Z, P]
        lib.attn_bwd_workspace_bytes.restype = Z
        lib.attn_bwd_workspace_bytes.argtypes = [I, I, I]
        lib.attn_decode.restype = I
        lib.attn_decode.argtypes = [I, I, I, I, I, I, I, P, P, P, I, F, F, I, I, I, P, P, P, I, P, Z, P]
        lib.attn_decode_noalloc.restype = I
        lib.attn_decode_noalloc.argtypes = [I, I, I, I, I, I, I, P, P, P, I, F, F, I, I, I, P, P, P, I, P]
        lib.attn_decode_num_splits.restype = I
        lib.attn_decode_num_splits.argtypes = [I] * 8
        lib.attn_decode_workspace_bytes.restype = Z
        lib.attn_decode_workspace_bytes.argtypes = [I] * 9
        LL = ctypes.c_longlong
        lib.attn_stream_append.restype = I
        lib.attn_stream_append.argtypes = [I, I, I, I, I, I, LL, I, P, P, P, P, P]
        lib.attn_stream_decode.restype = I
        lib.attn_stream_decode.argtypes = [I, I, I, I, I, I, I, LL, P, P, P, I, F, F, P, P, P, I, P, Z, P]
        lib.attn_stream_decode_workspace_bytes.restype = Z
        lib.attn_stream_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, LL, I]
        lib.attn_socket_code_bytes.restype = I
        lib.attn_socket_code_bytes.argtypes = [I, I]
        lib.attn_socket_hash.restype = I
        lib.attn_socket_hash.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P]
        lib.attn_socket_decode.restype = I
        lib.attn_socket_decode.argtypes = [I, I, I, I, I, I, I, I, F, I, P, P, P, P, P, P, I, F, F, P, P, P, P, I, P,
                                           Z, P]
        lib.attn_socket_decode_workspace_bytes.restype = Z
        lib.attn_socket_decode_workspace_bytes.argtypes = [I] * 9
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [I]
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_probe_sink_words.restype = Z
        lib.attn_probe_sink_words.argtypes = [Z]
        lib.attn_probe_read.restype = I
        lib.attn_probe_read.argtypes = [P, Z, P, P]
        lib.attn_probe_copy.restype = I
        lib.attn_probe_copy.argtypes = [P, P, Z, P]
        _lib = lib
    return _lib


def _check(rc: int) -> None:
    if rc != ATTN_OK:
        raise AttnError(rc, load().attn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported element type {t.dtype} (bfloat16 or float32)")


# Device type every tensor handed to the library must live on (the kernels dereference the
# pointers on the GPU; a host pointer would fault it).
_DEVICE_TYPE = "cuda"


def _check_like(name: str, t: Optional[torch.Tensor], shape, dtype, device) -> None:
    """Reject a caller-supplied tensor that the C ABI cannot size or type-check itself:
    wrong shape, element type, device, or a non-contiguous layout."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws: Optional[torch.Tensor], device) -> None:
    """A workspace is raw bytes: any element type, but contiguous and on the inputs' device
    (its size is checked by the library against the *_workspace_bytes query)."""
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")


def _common(q, k, v, sink, scale, mode, gamma):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device.type != _DEVICE_TYPE:
            raise ValueError(f"{name} must be on a GPU")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one element type")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    N, Hq, L, E = q.shape
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must have the same shape")
    if k.shape[0] != N or k.shape[3] != E:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in batch or head dimension")
    if sink is not None:
        if sink.dtype != torch.float32 or sink.device != q.device or not sink.is_contiguous() or sink.numel() != Hq:
            raise ValueError("sink must be a contiguous float32 tensor of Hq values on q's device")
    if mode not in MODES:
        raise ValueError(f"mode must be 'dot' or 'rbf', got {mode!r}")
    if scale is None:
        scale = 1.0 / math.sqrt(E)
    if gamma is None:
        gamma = 0.0
    return N, Hq, k.shape[1], L, k.shape[2], E, float(scale), float(gamma)


def _stream(dev: torch.device, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return s.cuda_stream


BIAS_NONE, BIAS_F32, BIAS_BOOL = 0, 1, 2


def _bias_args(bias: torch.Tensor, N: int, Hq: int, L: int, S: int, dev):
    """(kind, tensor, stride_n, stride_h) for a bias of shape (L, S) or (N or 1, Hq or 1, L, S)."""
    if bias.dim() == 2:
        bias = bias.reshape(1, 1, *bias.shape)
    if bias.dim() != 4 or tuple(bias.shape[2:]) != (L, S) or bias.shape[0] not in (1, N) or \
            bias.shape[1] not in (1, Hq):
        raise ValueError(f"bias {tuple(bias.shape)} does not broadcast to ({N}, {Hq}, {L}, {S})")
    if not bias.is_contiguous() or bias.device != dev:
        raise ValueError("bias must be contiguous and on q's device")
    if bias.dtype == torch.float32:
        kind = BIAS_F32
    elif bias.dtype in (torch.bool, torch.uint8):
        kind = BIAS_BOOL
        bias = bias.view(torch.uint8)
    else:
        raise TypeError(f"bias must be float32 (added to the logits) or bool (True = attend), got {bias.dtype}")
    sh = L * S if (bias.shape[1] == Hq and Hq > 1) else 0
    sn = bias.shape[1] * L * S if (bias.shape[0] == N and N > 1) else 0
    return kind, bias, sn, sh


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
        mode: str = "dot", gamma: Optional[float] = None, causal: bool = False, window: int = 0,
        n_reg: int = 0, sink: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
        key_len: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward through attn_fwd (or attn_fwd_biased when a bias or key lengths are given);
    returns (o, lse).  bias: float32 addend or bool mask (True = attend), shape (L, S) or
    (N or 1, Hq or 1, L, S); key_len: (N,) int32, real keys past key_len[n] are padding."""
    N, Hq, Hkv, L, S, E, scale, gamma = _common(q, k, v, sink, scale, mode, gamma)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (N, Hq, L), torch.float32, q.device)
    kind, bt, sn, sh = (BIAS_NONE, None, 0, 0) if bias is None else _bias_args(bias, N, Hq, L, S, q.device)
    if key_len is not None:
        if not isinstance(key_len, torch.Tensor) or key_len.dtype != torch.int32 or key_len.numel() != N or \
                key_len.device != q.device or not key_len.is_contiguous():
            raise ValueError("key_len must be a contiguous int32 tensor of N values on q's device")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((N, Hq, L), dtype=torch.float32, device=q.device)
    lib = load()
    if bias is None and key_len is None:
        rc = lib.attn_fwd(_dtype_code(q), N, Hq, Hkv, L, S, E, _ptr(q), _ptr(k), _ptr(v), MODES[mode],
                          scale, gamma, int(bool(causal)), int(window), int(n_reg), _ptr(sink),
                          _ptr(out), _ptr(lse), _stream(q.device, stream))
        _check(rc)
        return out, lse
    rc = lib.attn_fwd_biased(_dtype_code(q), N, Hq, Hkv, L, S, E, _ptr(q), _ptr(k), _ptr(v), MODES[mode],
                             scale, gamma, int(bool(causal)), int(window), int(n_reg), _ptr(sink),
                             kind, _ptr(bt), sn, sh, _ptr(key_len), _ptr(out), _ptr(lse),
                             _stream(q.device, stream))
    _check(rc)
    return out, lse


def decode_num_splits(N: int, Hq: int, Hkv: int, S: int, E: int, causal: bool = True, window: int = 0,
                      n_reg: int = 0) -> int:
    r = load().attn_decode_num_splits(N, Hq, Hkv, S, E, int(bool(causal)), window, n_reg)
    _check(min(r, 0))
    return r


def decode_workspace_bytes(N: int, Hq: int, Hkv: int, S: int, E: int, causal: bool = True, window: int = 0,
                           n_reg: int = 0, num_splits: int = 0) -> int:
    return int(load().attn_decode_workspace_bytes(N, Hq, Hkv, S, E, int(bool(causal)), window, n_reg,
                                                  num_splits))


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
           mode: str = "dot", gamma: Optional[float] = None, causal: bool = True, window: int = 0,
           n_reg: int = 0, sink: Optional[torch.Tensor] = None, num_splits: int = 0,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-K decode (q has L == 1) through attn_decode; returns (o, lse)."""
    N, Hq, Hkv, L, S, E, scale, gamma = _common(q, k, v, sink, scale, mode, gamma)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (N, Hq, L), torch.float32, q.device)
    _check_workspace(workspace, q.device)
    need = decode_workspace_bytes(N, Hq, Hkv, S, E, causal, window, n_reg, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((N, Hq, L), dtype=torch.float32, device=q.device)
    lib = load()
    rc = lib.attn_decode(_dtype_code(q), N, Hq, Hkv, L, S, E, _ptr(q), _ptr(k), _ptr(v), MODES[mode],
                         scale, gamma, int(bool(causal)), int(window), int(n_reg), _ptr(sink),
                         _ptr(out), _ptr(lse), int(num_splits), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(q.device, stream))
    _check(rc)
    return out, lse


DECODE_NOALLOC_SCRATCH_BYTES = 8 << 20  # ATTN_DECODE_NOALLOC_SCRATCH_BYTES of include/attn.h


def decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
                   mode: str = "dot", gamma: Optional[float] = None, causal: bool = True, window: int = 0,
                   n_reg: int = 0, sink: Optional[torch.Tensor] = None, num_splits: int = 0,
                   out: torch.Tensor, lse: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-K decode through attn_decode_noalloc: like decode, but the split partials go to
    the library's static device scratch (no workspace, no allocation by the library or
    here: out and lse must be given).  Calls that overlap on one GPU race."""
    N, Hq, Hkv, L, S, E, scale, gamma = _common(q, k, v, sink, scale, mode, gamma)
    if out is None or lse is None:
        raise ValueError("decode_noalloc needs out and lse (it allocates nothing)")
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (N, Hq, L), torch.float32, q.device)
    rc = load().attn_decode_noalloc(_dtype_code(q), N, Hq, Hkv, L, S, E, _ptr(q), _ptr(k), _ptr(v), MODES[mode],
                                    scale, gamma, int(bool(causal)), int(window), int(n_reg), _ptr(sink),
                                    _ptr(out), _ptr(lse), int(num_splits), _stream(q.device, stream))
    _check(rc)
    return out, lse


def _cache_check(k_cache, v_cache, n_sink: int, window: int):
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_contiguous() or t.device.type != _DEVICE_TYPE:
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.device != v_cache.device:
        raise ValueError("k_cache and v_cache must match in shape, element type and device")
    if k_cache.shape[2] != n_sink + window:
        raise ValueError(f"cache has {k_cache.shape[2]} rows per head, expected n_sink + window = {n_sink + window}")


def stream_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *,
                  n_sink: int, window: int, pos: int, stream=None) -> None:
    """Write the tokens at positions pos .. pos+T-1 (k_new, v_new: (N, Hkv, T, E)) into the rolling
    cache (N, Hkv, n_sink + window, E) through attn_stream_append."""
    _cache_check(k_cache, v_cache, n_sink, window)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_contiguous() or t.device != k_cache.device or t.dtype != k_cache.dtype:
            raise ValueError(f"{name} must be a contiguous 4-D tensor like the cache")
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have the same shape")
    N, Hkv, T, E = k_new.shape
    if (k_cache.shape[0], k_cache.shape[1], k_cache.shape[3]) != (N, Hkv, E):
        raise ValueError(f"new tokens {tuple(k_new.shape)} do not match the cache {tuple(k_cache.shape)}")
    rc = load().attn_stream_append(_dtype_code(k_new), N, Hkv, E, int(n_sink), int(window), int(pos), T,
                                   _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                   _stream(k_new.device, stream))
    _check(rc)


def stream_decode_workspace_bytes(N: int, Hq: int, Hkv: int, E: int, n_sink: int, window: int, pos: int,
                                  num_splits: int = 0) -> int:
    return int(load().attn_stream_decode_workspace_bytes(N, Hq, Hkv, E, n_sink, window, pos, num_splits))


def stream_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *, n_sink: int, window: int,
                  pos: int, scale: Optional[float] = None, mode: str = "dot", gamma: Optional[float] = None,
                  sink: Optional[torch.Tensor] = None, num_splits: int = 0,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode of the token at position `pos` (q: (N, Hq, 1, E)) against every token the rolling
    cache keeps, through attn_stream_decode; returns (o, lse)."""
    _cache_check(k_cache, v_cache, n_sink, window)
    N, Hq, Hkv, L, _, E, scale, gamma = _common(q, k_cache, v_cache, sink, scale, mode, gamma)
    if L != 1:
        raise ValueError(f"stream_decode takes one query per sequence, got q {tuple(q.shape)}")
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (N, Hq, L), torch.float32, q.device)
    _check_workspace(workspace, q.device)
    need = stream_decode_workspace_bytes(N, Hq, Hkv, E, n_sink, window, pos, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((N, Hq, L), dtype=torch.float32, device=q.device)
    rc = load().attn_stream_decode(_dtype_code(q), N, Hq, Hkv, E, int(n_sink), int(window), int(pos),
                                   _ptr(q), _ptr(k_cache), _ptr(v_cache), MODES[mode], scale, gamma, _ptr(sink),
                                   _ptr(out), _ptr(lse), int(num_splits), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(q.device, stream))
    _check(rc)
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, scale: Optional[float] = None, mode: str = "dot", gamma: Optional[float] = None,
        causal: bool = False, window: int = 0, n_reg: int = 0, sink: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients of fwd's o (for the upstream gradient dout) through attn_bwd.
    Returns (dq, dk, dv, dsink); dsink is None without a sink."""
    N, Hq, Hkv, L, S, E, scale, gamma = _common(q, k, v, sink, scale, mode, gamma)
    for name, t in (("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    _check_like("lse", lse, (N, Hq, L), torch.float32, q.device)
    _check_workspace(workspace, q.device)
    lib = load()
    need = int(lib.attn_bwd_workspace_bytes(N, Hq, L))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsink = torch.empty(Hq, dtype=torch.float32, device=q.device) if sink is not None else None
    rc = lib.attn_bwd(_dtype_code(q), N, Hq, Hkv, L, S, E, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                      MODES[mode], scale, gamma, int(bool(causal)), int(window), int(n_reg), _ptr(sink),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _stream(q.device, stream))
    _check(rc)
    return dq, dk, dv, dsink


def socket_code_bytes(tables: int, bits: int) -> int:
    """Bytes of bucket codes per key (attn_socket_code_bytes)."""
    r = load().attn_socket_code_bytes(int(tables), int(bits))
    _check(min(r, 0))
    return r


def unpack_codes(buckets: torch.Tensor, tables: int, bits: int) -> torch.Tensor:
    """Bucket codes (..., C) as stored by socket_hash -> one code per table (..., tables) uint8."""
    if bits > 4:
        return buckets[..., :tables]
    lo, hi = buckets & 15, buckets >> 4
    return torch.stack((lo, hi), dim=-1).flatten(-2)[..., :tables]


def socket_hash(k: torch.Tensor, v: torch.Tensor, proj: torch.Tensor, *, tables: int, bits: int,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """SOCKET prefill hashing through attn_socket_hash: bucket codes (N, Hkv, S, C) uint8 with
    C = socket_code_bytes(tables, bits) (codes of at most 4 bits packed two per byte, see
    unpack_codes) and value norms (N, Hkv, S) float32 of a bf16 or float32 key/value cache; proj
    (tables*bits, E) float32."""
    for name, t in (("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_contiguous() or \
                t.device.type != _DEVICE_TYPE:
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor")
    if k.shape != v.shape or k.dtype != v.dtype or k.device != v.device:
        raise ValueError("k and v must match in shape, element type and device")
    _check_like("proj", proj, (tables * bits, k.shape[3]), torch.float32, k.device)
    N, Hkv, S, E = k.shape
    buckets = torch.empty((N, Hkv, S, socket_code_bytes(tables, bits)), dtype=torch.uint8, device=k.device)
    vnorm = torch.empty((N, Hkv, S), dtype=torch.float32, device=k.device)
    rc = load().attn_socket_hash(_dtype_code(k), N, Hkv, S, E, int(tables), int(bits), _ptr(k), _ptr(v),
                                 _ptr(proj), _ptr(buckets), _ptr(vnorm), _stream(k.device, stream))
    _check(rc)
    return buckets, vnorm


def socket_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, proj: torch.Tensor, buckets: torch.Tensor,
                  vnorm: torch.Tensor, *, tables: int, bits: int, tau: float, top_k: int,
                  scale: Optional[float] = None, mode: str = "dot", gamma: Optional[float] = None,
                  sink: Optional[torch.Tensor] = None, num_splits: int = 0, want_selected: bool = False,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, stream=None):
    """SOCKET sparse decode through attn_socket_decode; returns (o, lse, selected or None)."""
    N, Hq, Hkv, L, S, E, scale, gamma = _common(q, k, v, sink, scale, mode, gamma)
    if L != 1:
        raise ValueError(f"socket_decode takes one query per sequence, got q {tuple(q.shape)}")
    _check_like("proj", proj, (tables * bits, E), torch.float32, q.device)
    _check_like("buckets", buckets, (N, Hkv, S, socket_code_bytes(tables, bits)), torch.uint8, q.device)
    _check_like("vnorm", vnorm, (N, Hkv, S), torch.float32, q.device)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (N, Hq, 1), torch.float32, q.device)
    _check_workspace(workspace, q.device)
    lib = load()
    need = int(lib.attn_socket_decode_workspace_bytes(N, Hq, Hkv, S, E, tables, bits, top_k, num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((N, Hq, 1), dtype=torch.float32, device=q.device)
    sel = torch.empty((N, Hq, top_k), dtype=torch.int32, device=q.device) if want_selected else None
    rc = lib.attn_socket_decode(_dtype_code(q), N, Hq, Hkv, S, E, int(tables), int(bits), float(tau), int(top_k),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(proj), _ptr(buckets), _ptr(vnorm), MODES[mode],
                                scale, gamma, _ptr(sink), _ptr(out), _ptr(lse), _ptr(sel), int(num_splits),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(q.device, stream))
    _check(rc)
    return out, lse, sel


# ----------------------------------------------------------------------------- bandwidth probes


def _probe_buffer(name: str, t: torch.Tensor) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_contiguous() or t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t.numel() * t.element_size()


def probe_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Stream src once through attn_probe_read (include/attn_probe.h); returns the sink words."""
    nbytes = _probe_buffer("src", src)
    lib = load()
    if sink is None:
        sink = torch.empty(max(int(lib.attn_probe_sink_words(nbytes)), 1), dtype=torch.int32, device=src.device)
    _check(lib.attn_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(src.device, stream)))
    return sink


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Copy src into dst (same byte size) through attn_probe_copy."""
    nbytes = _probe_buffer("src", src)
    if _probe_buffer("dst", dst) != nbytes or dst.device != src.device:
        raise ValueError("dst must be a GPU tensor of src's byte size on src's device")
    _check(load().attn_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(src.device, stream)))
