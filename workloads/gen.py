"""Seeded synthetic inputs for the attention workloads.

This module draws random tensors and rounds them to the storage type; it holds
none of the attention arithmetic.  Both the fp64 oracle and the GPU library are
fed from here: the oracle reads the returned host arrays, the GPU receives the
same bits by a host-to-device copy.

Recipe (one numpy PCG64 stream per tensor slice, so any slice can be redrawn
on its own without drawing the rest):

* slice (tensor t, batch n, head h) uses ``SeedSequence([seed, t, n, h])``
  with t = 0 for Q, 1 for K, 2 for V;
* Q, V and (k_dist="normal") K: iid N(0, 1) drawn in float32;
* K with k_dist="dir_lognormal": a direction g/|g| with g ~ N(0, I_E) (float64)
  times a per-token magnitude exp(N(0, 1)), so |k| is lognormal(0, 1);
* register tokens (the first n_reg rows of K and V): keys are exactly zero,
  values N(0, 0.02**2) drawn once per head from ``SeedSequence([seed, 3, h])``
  and shared by every batch entry;
* sink logits: Hq values N(0, 1) in float32 from ``SeedSequence([seed, 4])``;
* "bf16" tensors are the float32 draws rounded to nearest-even bfloat16 and
  returned as uint16 bit patterns; "f32" tensors are the float32 draws.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Workload

T_Q, T_K, T_V, T_REG, T_SINK = 0, 1, 2, 3, 4


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(u: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for test-side inspection)."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def q_slice(w: Workload, n: int, h: int) -> np.ndarray:
    x = _rng(w.seed, T_Q, n, h).standard_normal((w.L, w.E), dtype=np.float32)
    return _store(x, w.dtype)


def _real_keys_f32(w: Workload, n: int, h: int) -> np.ndarray:
    rng = _rng(w.seed, T_K, n, h)
    if w.k_dist == "normal":
        return rng.standard_normal((w.S_real, w.E), dtype=np.float32)
    if w.k_dist == "dir_lognormal":
        g = rng.standard_normal((w.S_real, w.E))
        g /= np.sqrt(np.sum(g * g, axis=1, keepdims=True))
        mag = np.exp(rng.standard_normal(w.S_real))
        return (g * mag[:, None]).astype(np.float32)
    raise ValueError(f"unknown k_dist {w.k_dist!r}")


def register_values_f32(w: Workload, h: int) -> np.ndarray:
    return (_rng(w.seed, T_REG, h).standard_normal((w.n_reg, w.E)) * 0.02).astype(np.float32)


def k_slice(w: Workload, n: int, h: int) -> np.ndarray:
    x = np.zeros((w.S, w.E), dtype=np.float32)
    x[w.n_reg:] = _real_keys_f32(w, n, h)
    return _store(x, w.dtype)


def v_slice(w: Workload, n: int, h: int) -> np.ndarray:
    x = np.empty((w.S, w.E), dtype=np.float32)
    if w.n_reg:
        x[:w.n_reg] = register_values_f32(w, h)
    x[w.n_reg:] = _rng(w.seed, T_V, n, h).standard_normal((w.S_real, w.E), dtype=np.float32)
    return _store(x, w.dtype)


def sink_logits(w: Workload) -> Optional[np.ndarray]:
    if not w.sink:
        return None
    return _rng(w.seed, T_SINK).standard_normal(w.Hq, dtype=np.float32)


@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray                # (N,Hq,L,E) uint16 bf16 bits or float32
    k: np.ndarray                # (N,Hkv,S,E)
    v: np.ndarray                # (N,Hkv,S,E)
    sink: Optional[np.ndarray]   # (Hq,) float32 or None
    bias: Optional[np.ndarray] = None     # general bias (N|1, Hq|1, L, S): float32 or bool, or None
    key_len: Optional[np.ndarray] = None  # (N,) int32 valid real keys, or None


def _default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(w: Workload, threads: Optional[int] = None) -> Inputs:
    """Draw every tensor of workload ``w`` (slice by slice, in a thread pool)."""
    st = np.uint16 if w.dtype == "bf16" else np.float32
    q = np.empty((w.N, w.Hq, w.L, w.E), dtype=st)
    k = np.empty((w.N, w.Hkv, w.S, w.E), dtype=st)
    v = np.empty((w.N, w.Hkv, w.S, w.E), dtype=st)
    jobs = []
    for n in range(w.N):
        for h in range(w.Hq):
            jobs.append((q, q_slice, n, h))
        for h in range(w.Hkv):
            jobs.append((k, k_slice, n, h))
            jobs.append((v, v_slice, n, h))

    def run(job):
        dst, fn, n, h = job
        dst[n, h] = fn(w, n, h)

    nthr = threads or _default_threads()
    if nthr <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(run, jobs))
    bias = None
    if w.bias != "none":
        shape = (w.N if w.bias_dims[0] == "N" else 1, w.Hq if w.bias_dims[1] == "H" else 1, w.L, w.S)
        bias = bias_f32(w.seed, shape) if w.bias == "f32" else mask_bool(w.seed, shape, 0.9)
    key_len = np.asarray(w.key_len, dtype=np.int32) if w.key_len else None
    return Inputs(w, q, k, v, sink_logits(w), bias, key_len)


# ----------------------------------------------------------------------------- general bias inputs


def bias_f32(seed: int, shape, scale: float = 1.0, p_neg_inf: float = 0.0) -> np.ndarray:
    """Float32 bias N(0, scale); a fraction p_neg_inf of the entries is -inf (hidden pairs)."""
    r = _rng(seed, 7)
    b = (r.standard_normal(shape) * scale).astype(np.float32)
    if p_neg_inf > 0.0:
        b[r.random(shape) < p_neg_inf] = -np.inf
    return b


def mask_bool(seed: int, shape, p_keep: float) -> np.ndarray:
    """Boolean mask (True = the pair is used) with each entry kept with probability p_keep."""
    return _rng(seed, 8).random(shape) < p_keep


def key_lengths(seed: int, N: int, S_real: int) -> np.ndarray:
    """Per-sequence valid key counts in [0, S_real] (int32); the first one is always S_real."""
    k = _rng(seed, 9).integers(0, S_real + 1, size=N).astype(np.int32)
    k[0] = S_real
    return k


def socket_projections(seed: int, tables: int, bits: int, E: int) -> np.ndarray:
    """Random hyperplanes for SOCKET hashing: (tables*bits, E) float32, iid N(0, 1)."""
    return _rng(seed, 10).standard_normal((tables * bits, E)).astype(np.float32)
