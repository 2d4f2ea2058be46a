"""The five synthetic attention workloads, as plain data.

Each workload is one call of the attention forward (or decode) with the shapes,
distributions and flags listed below.  Nothing here computes attention; this
module only names sizes and flags so that the generator, the oracle, the tests
and the benchmark agree on them.

Sources (the pages): shapes Q (N,Hq,L,E) and K/V (N,H,S,E) follow the SDPA
problem statement ("SDPA란 무엇인가?", section 1); the RBF logit and register
tokens follow the RBF-attention digest ("Dot-Product Attention을 거리 기반
RBF-Attention으로 교체한 실험기", section details paragraphs 2-4); the per-head
sink logit follows "Attention Sink" section 4.2; the 100K+ token decode regime
follows the SOCKET summary (results).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" or "f32": element type of Q, K, V and O
    N: int                # batch
    Hq: int               # query heads
    Hkv: int              # key/value heads (Hq % Hkv == 0)
    L: int                # query length
    S_real: int           # real keys (registers not included)
    E: int                # head dimension (E_v == E)
    mode: str             # "dot" or "rbf"
    scale: float          # dot mode logit scale (ignored in rbf mode)
    gamma: float          # rbf mode gamma (ignored in dot mode)
    causal: bool
    window: int           # 0 = no window
    n_reg: int            # register tokens prepended to K/V
    sink: bool            # per-query-head sink logit present
    decode: bool          # uses the split-K decode entry point (L == 1)
    seed: int
    k_dist: str = "normal"  # "normal" or "dir_lognormal"
    bias: str = "none"      # general bias: "none", "f32" (N(0,1) addend) or "bool" (mask)
    bias_dims: str = "11"   # bias batch / head dims: "N" or "1", then "H" or "1"
    key_len: tuple = ()     # per-sequence valid real keys (empty: no padding)

    @property
    def S(self) -> int:
        return self.S_real + self.n_reg

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


C1 = Workload("rbf_causal_f32_1x1x256x64", "f32", 1, 1, 1, 256, 256, 64,
              "rbf", 1.0 / 8.0, 1.0 / 8.0, True, 0, 0, False, False, 1)
C2 = Workload("dot_causal_bf16_4x16x2048x128", "bf16", 4, 16, 16, 2048, 2048, 128,
              "dot", 1.0 / math.sqrt(128.0), 0.0, True, 0, 0, False, False, 2)
C3 = Workload("rbf_causal_reg4_bf16_2x16x8192x64", "bf16", 2, 16, 16, 8192, 8192, 64,
              "rbf", 1.0 / 8.0, 1.0 / 8.0, True, 0, 4, False, False, 3,
              k_dist="dir_lognormal")
C4 = Workload("sink_swa128_gqa64to8_bf16_1x8192x64", "bf16", 1, 64, 8, 8192, 8192, 64,
              "dot", 1.0 / 8.0, 0.0, True, 128, 0, True, False, 4)
C5 = Workload("decode_splitk_sink_bf16_8x32to8x131072x128", "bf16", 8, 32, 8, 1, 131072, 128,
              "dot", 1.0 / math.sqrt(128.0), 0.0, True, 0, 0, True, True, 5)

ALL = (C1, C2, C3, C4, C5)

# The headline prefill shape with the SDPA page's general bias: a float32 bias
# per sequence (broadcast over heads) added to the logits, and key padding
# (right-padded sequences of 2048, 1792, 1536 and 1024 valid keys).
B1 = Workload("dot_causal_bias_keypad_bf16_4x16x2048x128", "bf16", 4, 16, 16, 2048, 2048, 128,
              "dot", 1.0 / math.sqrt(128.0), 0.0, True, 0, 0, False, False, 7,
              bias="f32", bias_dims="N1", key_len=(2048, 1792, 1536, 1024))
EXTRA = (B1,)
BY_NAME = {w.name: w for w in ALL + EXTRA}


def visible_pairs_per_head(w: Workload, key_len: int = -1) -> int:
    """Count (query, key) pairs that the visibility rule lets through, per head.

    Register keys are always visible; real key r is visible to query i (aligned
    bottom-right, i' = i + S_real - L) iff (not causal or r <= i') and
    (window <= 0 or i' - r < window), and r < key_len when a sequence's key
    length is given.  Closed-form per query row.
    """
    total = 0
    off = w.S_real - w.L
    kl = w.S_real if key_len < 0 else min(w.S_real, key_len)
    for i in range(w.L):
        ip = i + off
        hi = min(kl - 1, ip) if w.causal else kl - 1
        lo = max(0, ip - w.window + 1) if w.window > 0 else 0
        total += max(0, hi - lo + 1) + w.n_reg
    return total


def algorithmic_flops(w: Workload) -> float:
    """4*E flops per visible pair (2E for q.k, 2E for p*v), times the heads; with key
    lengths, each sequence counts its own pairs (padding and a user bias's -inf
    entries are not credited; the f32 bias here has none)."""
    if w.key_len:
        return 4.0 * w.E * w.Hq * sum(visible_pairs_per_head(w, kl) for kl in w.key_len)
    return 4.0 * w.E * visible_pairs_per_head(w) * w.N * w.Hq


def algorithmic_bytes(w: Workload) -> float:
    """Each tensor touched once: Q, K, V read, O written, LSE written, sink read."""
    esz = 2 if w.dtype == "bf16" else 4
    q = w.N * w.Hq * w.L * w.E * esz
    kv = 2 * w.N * w.Hkv * w.S * w.E * esz
    o = q
    lse = w.N * w.Hq * w.L * 4
    sink = w.Hq * 4 if w.sink else 0
    bias = 0
    if w.bias != "none":
        bias = ((w.N if w.bias_dims[0] == "N" else 1) * (w.Hq if w.bias_dims[1] == "H" else 1) * w.L * w.S *
                (4 if w.bias == "f32" else 1))
    return float(q + kv + o + lse + sink + bias + 4 * len(w.key_len))


@dataclass(frozen=True)
class StreamWorkload:
    """One step of streaming decode over a rolling (StreamingLLM) cache: append the
    newest token's key/value, then decode its query against the n_sink first
    tokens and the `window` most recent ones ("Attention Sink LLM..." page,
    section 3.2).  `pos` is the newest token's absolute position; the cache
    holds n_sink + window rows per (batch, kv head)."""
    name: str
    N: int
    Hq: int
    Hkv: int
    E: int
    n_sink: int
    window: int
    pos: int
    sink: bool
    seed: int
    mode: str = "dot"
    scale: float = 0.0
    gamma: float = 0.0
    dtype: str = "bf16"

    @property
    def rows(self) -> int:
        return min(self.pos + 1, self.n_sink + self.window)


# StreamingLLM-sized cache (4 sink tokens + a 4092-token window) deep into a
# stream, with the long-context decode shape's heads (32 query over 8 kv heads).
STREAM1 = StreamWorkload("stream_sink4_win4092_bf16_8x32to8x128_pos100000", 8, 32, 8, 128, 4, 4092, 100000,
                         True, 6, scale=1.0 / math.sqrt(128.0))
STREAM_BY_NAME = {STREAM1.name: STREAM1}


def stream_bytes(w: StreamWorkload) -> float:
    """Per step: the new token's key/value read and written once, every kept row of
    the cache read once, q read, o and lse written, sink read."""
    esz = 2
    new = 2 * w.N * w.Hkv * w.E * esz
    kv = 2 * w.N * w.Hkv * w.rows * w.E * esz
    q = w.N * w.Hq * w.E * esz
    return float(2 * new + kv + 2 * q + w.N * w.Hq * 4 + (w.Hq * 4 if w.sink else 0))


# Backward steps measured on the prefill shapes C2 and C3 (gradients of O for a
# seeded upstream gradient).
BACKWARD = (C2, C3)


def backward_flops(w: Workload) -> float:
    """10*E flops per visible pair: the logits recomputed once (2E) and the four
    gradient products dP = dO V^T, dV = P^T dO, dK = dS^T Q, dQ = dS K (2E each)."""
    return 2.5 * algorithmic_flops(w)


def backward_bytes(w: Workload) -> float:
    """Q, K, V, O, dO read once; dQ, dK, dV written once; LSE read."""
    esz = 2 if w.dtype == "bf16" else 4
    qo = w.N * w.Hq * w.L * w.E * esz
    kv = w.N * w.Hkv * w.S * w.E * esz
    return float(3 * qo + 2 * kv + qo + 2 * kv + w.N * w.Hq * w.L * 4)


@dataclass(frozen=True)
class SocketWorkload:
    """One SOCKET sparse decode step ("기술 요약: SOCKET" page, method): score every key of the
    cache by soft collisions, select top_k per query head, attend to them exactly.  The
    cache and queries are those of `base` (a decode workload); hashing is prefill work and
    is not part of the step."""
    name: str
    base: Workload
    tables: int
    bits: int
    tau: float
    top_k: int


# The long-context decode shape at about 33x sparsity (the page's setting), 64 tables of
# 4-bit codes (32 bytes of packed codes + a 4-byte norm per key: 7% of the K and V bytes).
SOCKET1 = SocketWorkload("socket_decode_sink_bf16_8x32to8x131072x128_k3972", C5, 64, 4, 4.0, 3972)
SOCKET_BY_NAME = {SOCKET1.name: SOCKET1}


def socket_code_bytes(tables: int, bits: int) -> int:
    """Bytes of bucket codes per key: codes of at most 4 bits are stored two per byte."""
    return (tables + 1) // 2 if bits <= 4 else tables


def socket_bytes(sw: SocketWorkload) -> float:
    """Per step: every key's codes and value norm read once per kv head, the selected K and V
    rows read once per query head, q read and o / lse written."""
    w = sw.base
    keys = w.N * w.Hkv * w.S
    return float(keys * (socket_code_bytes(sw.tables, sw.bits) + 4) + 2 * w.N * w.Hq * sw.top_k * w.E * 2 +
                 2 * w.N * w.Hq * w.E * 2 + w.N * w.Hq * 4)
