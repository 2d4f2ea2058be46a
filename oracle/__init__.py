"""fp64 CPU oracle for softmax attention (ctypes binding of attn_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use it.  The GPU library never imports it, and this
package never imports the GPU library.

The definition it computes, with the page citations, is in attn_oracle.h.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")

BF16, F32, F64 = 0, 1, 2
DOT, RBF = 0, 1

_default = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle C source with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-Wextra", "-I", _HERE, "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def bind(path: str):
    """Load an oracle shared library built by build(); returns a handle for attn(lib=...)."""
    return _bind(path)


def _bind(path: str):
    lib = ctypes.CDLL(path)
    vp, dp, llp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong)
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, vp, vp, ctypes.c_int, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, dp,
        ctypes.c_longlong, llp, dp, dp, dp, ctypes.c_int]
    lib.oracle_attn_rows_ex.restype = ctypes.c_int
    lib.oracle_attn_rows_ex.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, vp, vp, ctypes.c_int, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, dp,
        ctypes.c_int, vp, ctypes.c_longlong, ctypes.c_longlong, ctypes.POINTER(ctypes.c_int),
        ctypes.c_longlong, llp, dp, dp, dp, ctypes.c_int]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, vp, vp, vp, ctypes.c_int, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, dp,
        ctypes.c_longlong, llp, dp, ctypes.c_longlong, llp, dp, dp, dp, dp, dp, ctypes.c_int]
    u8p = ctypes.POINTER(ctypes.c_ubyte)
    fp = ctypes.POINTER(ctypes.c_float)
    lib.oracle_socket_hash.restype = ctypes.c_int
    lib.oracle_socket_hash.argtypes = [ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       vp, vp, fp, u8p, dp]
    lib.oracle_socket_scores.restype = ctypes.c_int
    lib.oracle_socket_scores.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         vp, fp, ctypes.c_longlong, u8p, dp, dp]
    lib.oracle_socket_select.restype = ctypes.c_int
    lib.oracle_socket_select.argtypes = [ctypes.c_longlong, dp, ctypes.c_longlong, llp]
    lib.oracle_visible.restype = ctypes.c_int
    lib.oracle_visible.argtypes = [ctypes.c_int] * 7
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _default = _bind(_LIB)
    return _default


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle: unsupported element type {a.dtype}")


def visible(L: int, S: int, causal: bool, window: int, n_reg: int, i: int, j: int, lib=None) -> bool:
    return bool((lib or _load()).oracle_visible(L, S, int(causal), window, n_reg, i, j))


def num_threads(threads: int = 0, lib=None) -> int:
    return (lib or _load()).oracle_num_threads(threads)


BIAS_NONE, BIAS_F32, BIAS_BOOL = 0, 1, 2


def bias_strides(bias: np.ndarray, N: int, Hq: int, L: int, S: int):
    """Element strides (batch, head) of a bias of shape (N or 1, Hq or 1, L, S); 0 = broadcast."""
    if bias.ndim != 4 or bias.shape[2:] != (L, S) or bias.shape[0] not in (1, N) or bias.shape[1] not in (1, Hq):
        raise ValueError(f"bias shape {bias.shape} does not broadcast to ({N}, {Hq}, {L}, {S})")
    sh = L * S if (bias.shape[1] == Hq and Hq > 1) else 0
    sn = bias.shape[1] * L * S if (bias.shape[0] == N and N > 1) else 0
    return sn, sh


def attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, mode: str = "dot", scale: Optional[float] = None,
         gamma: float = 0.0, causal: bool = False, window: int = 0, n_reg: int = 0,
         sink: Optional[np.ndarray] = None, bias: Optional[np.ndarray] = None,
         key_len: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None,
         want_p: bool = False, threads: int = 0, lib=None):
    """Attention rows in fp64.

    q (N,Hq,L,E), k and v (N,Hkv,S,E): uint16 (bf16 bits), float32 or float64,
    all the same type.  rows: flat indices (n*Hq+h)*L+i, or None for all rows.
    bias: None, a float32 additive bias or a bool mask (True = use the pair),
    shape (N or 1, Hq or 1, L, S).  key_len: None or N valid real-key counts.
    Returns (o, lse[, p]): o has shape (N,Hq,L,E) when rows is None, else
    (len(rows), E); lse matches without E; p has S columns.
    lib: a handle from bind() to use instead of the default build.
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("oracle: q, k, v must share one element type")
    N, Hq, L, E = q.shape
    Nk, Hkv, S, Ek = k.shape
    if v.shape != k.shape or Nk != N or Ek != E:
        raise ValueError("oracle: shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(E)
    md = {"dot": DOT, "rbf": RBF}[mode]
    sk = None
    if sink is not None:
        sk = np.ascontiguousarray(np.asarray(sink, dtype=np.float64).reshape(-1))
        if sk.shape[0] != Hq:
            raise ValueError("oracle: sink must hold Hq values")
    if rows is None:
        nrows = N * Hq * L
        rptr = None
        out_shape = (N, Hq, L)
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        nrows = rr.shape[0]
        rptr = rr.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong))
        out_shape = (nrows,)
    o = np.empty((nrows, E), dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64)
    p = np.empty((nrows, S), dtype=np.float64) if want_p else None
    dp = ctypes.POINTER(ctypes.c_double)
    kind, bptr, sn, sh = BIAS_NONE, None, 0, 0
    if bias is not None:
        if bias.dtype == np.float32:
            kind = BIAS_F32
            b = np.ascontiguousarray(bias)
        elif bias.dtype in (np.bool_, np.uint8):
            kind = BIAS_BOOL
            b = np.ascontiguousarray(bias.astype(np.uint8))
        else:
            raise TypeError("oracle: bias must be float32 or bool")
        sn, sh = bias_strides(b, N, Hq, L, S)
        bptr = b.ctypes.data
    kl = None
    if key_len is not None:
        kl = np.ascontiguousarray(np.asarray(key_len, dtype=np.int32).reshape(-1))
        if kl.shape[0] != N:
            raise ValueError("oracle: key_len must hold N values")
    rc = (lib or _load()).oracle_attn_rows_ex(
        dt, N, Hq, Hkv, L, S, E,
        q.ctypes.data, k.ctypes.data, v.ctypes.data, md, float(scale), float(gamma),
        int(bool(causal)), int(window), int(n_reg),
        sk.ctypes.data_as(dp) if sk is not None else None,
        kind, bptr, sn, sh, kl.ctypes.data_as(ctypes.POINTER(ctypes.c_int)) if kl is not None else None,
        nrows, rptr, o.ctypes.data_as(dp), lse.ctypes.data_as(dp),
        p.ctypes.data_as(dp) if p is not None else None, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows failed with code {rc}")
    o = o.reshape(out_shape + (E,))
    lse = lse.reshape(out_shape)
    if want_p:
        return o, lse, p.reshape(out_shape + (S,))
    return o, lse


def attn_workload(inp, rows: Optional[Sequence[int]] = None, want_p: bool = False, threads: int = 0):
    """Run the oracle on a workloads.gen.Inputs bundle (same flags as its workload)."""
    w = inp.workload
    return attn(inp.q, inp.k, inp.v, mode=w.mode, scale=w.scale, gamma=w.gamma, causal=w.causal,
                window=w.window, n_reg=w.n_reg, sink=inp.sink, bias=getattr(inp, "bias", None),
                key_len=getattr(inp, "key_len", None), rows=rows, want_p=want_p, threads=threads)


# ----------------------------------------------------------------------------- rolling (StreamingLLM) cache


def stream_kept_positions(n_sink: int, window: int, pos: int) -> np.ndarray:
    """Absolute positions a StreamingLLM cache holds once the token at `pos` is in it:
    the first n_sink tokens for good, plus the `window` most recent tokens ("Attention Sink
    LLM..." page, section 3.2: keep the initial tokens' KV, roll the recent ones)."""
    p = np.arange(pos + 1, dtype=np.int64)
    return p[(p < n_sink) | (p > pos - window)]


def stream_decode(q: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray, *, n_sink: int, window: int, pos: int,
                  mode: str = "dot", scale: Optional[float] = None, gamma: float = 0.0,
                  sink: Optional[np.ndarray] = None, threads: int = 0, lib=None):
    """Decode of the token at position `pos` over what the cache keeps.

    q (N,Hq,1,E); k_hist, v_hist (N,Hkv,>pos,E) with row p = the token at absolute
    position p.  The kept rows are gathered and attended to with no mask: every
    kept token precedes (or is) the query.  Returns (o (N,Hq,1,E), lse (N,Hq,1))."""
    kept = stream_kept_positions(n_sink, window, pos)
    k = np.ascontiguousarray(k_hist[:, :, kept])
    v = np.ascontiguousarray(v_hist[:, :, kept])
    return attn(q, k, v, mode=mode, scale=scale, gamma=gamma, causal=False, window=0, n_reg=0, sink=sink,
                threads=threads, lib=lib)


# ----------------------------------------------------------------------------- backward


def attn_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, *, mode: str = "dot",
             scale: Optional[float] = None, gamma: float = 0.0, causal: bool = False, window: int = 0,
             n_reg: int = 0, sink: Optional[np.ndarray] = None, qrows: Optional[Sequence[int]] = None,
             krows: Optional[Sequence[int]] = None, threads: int = 0, lib=None):
    """Gradients of O (for the upstream gradient dout, shaped like q) in fp64.

    Returns a dict: dq (N,Hq,L,E) or (len(qrows),E); dk, dv (N,Hkv,S,E) or
    (len(krows),E); dsink (Hq,) (zeros without a sink); lse, delta (N,Hq,L):
    the forward LSE and D_i = dO_i . O_i.  qrows: flat (n*Hq+h)*L+i;
    krows: flat (n*Hkv+kh)*S+j; None = all."""
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))
    dt = _dtype_code(q)
    if any(_dtype_code(a) != dt for a in (k, v, dout)):
        raise TypeError("oracle: q, k, v, dout must share one element type")
    N, Hq, L, E = q.shape
    _, Hkv, S, _ = k.shape
    if dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("oracle: shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(E)
    md = {"dot": DOT, "rbf": RBF}[mode]
    dp = ctypes.POINTER(ctypes.c_double)
    llp = ctypes.POINTER(ctypes.c_longlong)
    sk = None if sink is None else np.ascontiguousarray(np.asarray(sink, dtype=np.float64).reshape(-1))
    qr = None if qrows is None else np.ascontiguousarray(np.asarray(qrows, dtype=np.int64).reshape(-1))
    kr = None if krows is None else np.ascontiguousarray(np.asarray(krows, dtype=np.int64).reshape(-1))
    nq = N * Hq * L if qr is None else qr.shape[0]
    nk = N * Hkv * S if kr is None else kr.shape[0]
    dq = np.zeros((nq, E))
    dk = np.zeros((nk, E))
    dv = np.zeros((nk, E))
    dsink = np.zeros(Hq)
    lse = np.zeros(N * Hq * L)
    delta = np.zeros(N * Hq * L)
    rc = (lib or _load()).oracle_attn_bwd(
        dt, N, Hq, Hkv, L, S, E, q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
        md, float(scale), float(gamma), int(bool(causal)), int(window), int(n_reg),
        sk.ctypes.data_as(dp) if sk is not None else None,
        nq, qr.ctypes.data_as(llp) if qr is not None else None, dq.ctypes.data_as(dp),
        nk, kr.ctypes.data_as(llp) if kr is not None else None, dk.ctypes.data_as(dp), dv.ctypes.data_as(dp),
        dsink.ctypes.data_as(dp), lse.ctypes.data_as(dp), delta.ctypes.data_as(dp), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd failed with code {rc}")
    if qr is None:
        dq = dq.reshape(N, Hq, L, E)
    if kr is None:
        dk = dk.reshape(N, Hkv, S, E)
        dv = dv.reshape(N, Hkv, S, E)
    return {"dq": dq, "dk": dk, "dv": dv, "dsink": dsink, "lse": lse.reshape(N, Hq, L),
            "delta": delta.reshape(N, Hq, L)}


# ----------------------------------------------------------------------------- SOCKET sparse decode


def socket_hash(k: np.ndarray, v: np.ndarray, proj: np.ndarray, tables: int, bits: int, lib=None):
    """Bucket codes (N,Hkv,S,tables) uint8 and value norms (N,Hkv,S) fp64 of a key/value cache
    ("기술 요약: SOCKET" page, method step 1: keys hashed by random projections into L tables,
    value norms cached).  proj: (tables*bits, E) float32 hyperplanes."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    pr = np.ascontiguousarray(proj, dtype=np.float32)
    *lead, E = k.shape
    nkeys = int(np.prod(lead))
    buckets = np.zeros(nkeys * tables, dtype=np.uint8)
    vnorm = np.zeros(nkeys)
    rc = (lib or _load()).oracle_socket_hash(
        _dtype_code(k), nkeys, E, tables, bits, k.ctypes.data, v.ctypes.data,
        pr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), buckets.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)),
        vnorm.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_socket_hash failed with code {rc}")
    return buckets.reshape(*lead, tables), vnorm.reshape(lead)


def socket_scores(q_row: np.ndarray, proj: np.ndarray, buckets: np.ndarray, vnorm: np.ndarray, tables: int,
                  bits: int, tau: float, lib=None) -> np.ndarray:
    """Soft-collision scores of every key for one query row (method steps 2-3): the query's
    temperature softmax over each table's buckets, summed over the tables at each key's
    bucket, times the key's value norm.  buckets (S, tables), vnorm (S,)."""
    q_row = np.ascontiguousarray(q_row)
    pr = np.ascontiguousarray(proj, dtype=np.float32)
    b = np.ascontiguousarray(buckets, dtype=np.uint8)
    vn = np.ascontiguousarray(vnorm, dtype=np.float64)
    S = vn.shape[0]
    out = np.zeros(S)
    rc = (lib or _load()).oracle_socket_scores(
        _dtype_code(q_row), q_row.shape[-1], tables, bits, float(tau), q_row.ctypes.data,
        pr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), S, b.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)),
        vn.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_socket_scores failed with code {rc}")
    return out


def socket_select(scores: np.ndarray, top_k: int, lib=None) -> np.ndarray:
    """The top_k keys by score, ties to the lower index (method step 4: a deterministic
    top-k), returned in ascending key order."""
    sc = np.ascontiguousarray(scores, dtype=np.float64).reshape(-1)
    out = np.zeros(max(int(top_k), 0), dtype=np.int64)
    rc = (lib or _load()).oracle_socket_select(sc.shape[0], sc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                               int(top_k), out.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)))
    if rc != 0:
        raise ValueError(f"oracle_socket_select failed with code {rc}")
    return out


def socket_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, proj: np.ndarray, buckets: np.ndarray,
                  vnorm: np.ndarray, *, tables: int, bits: int, tau: float, top_k: int, mode: str = "dot",
                  scale: Optional[float] = None, gamma: float = 0.0, sink: Optional[np.ndarray] = None, lib=None):
    """Sparse decode of q (N,Hq,1,E): per query head, scores -> top_k -> exact attention over
    the selected keys (the same logits and sink as attn).  Returns (o (N,Hq,1,E), lse (N,Hq,1),
    selected (N,Hq,top_k) ascending key indices, scores (N,Hq,S))."""
    N, Hq, L, E = q.shape
    _, Hkv, S, _ = k.shape
    G = Hq // Hkv
    o = np.zeros((N, Hq, 1, E))
    lse = np.zeros((N, Hq, 1))
    sel = np.zeros((N, Hq, top_k), dtype=np.int64)
    sc = np.zeros((N, Hq, S))
    for n in range(N):
        for h in range(Hq):
            kh = h // G
            s = socket_scores(q[n, h, 0], proj, buckets[n, kh], vnorm[n, kh], tables, bits, tau, lib=lib)
            idx = socket_select(s, top_k, lib=lib)
            sc[n, h] = s
            sel[n, h] = idx
            kk = np.ascontiguousarray(k[n:n + 1, kh:kh + 1, idx])
            vv = np.ascontiguousarray(v[n:n + 1, kh:kh + 1, idx])
            sk = None if sink is None else np.asarray(sink, dtype=np.float64)[h:h + 1]
            oo, ll = attn(np.ascontiguousarray(q[n:n + 1, h:h + 1]), kk, vv, mode=mode, scale=scale, gamma=gamma,
                          sink=sk, lib=lib)
            o[n, h] = oo[0, 0]
            lse[n, h] = ll[0, 0]
    return o, lse, sel, sc
