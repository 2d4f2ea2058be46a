"""Helpers for the GPU parity tests: move generated inputs to the GPU, run the
library, run the oracle on the same bits, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import softmax_attention_attn_amd as attn
from workloads import gen
from workloads.configs import Workload

TOL_O = {"bf16": 2e-2, "f32": 1e-4}
TOL_LSE = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inp: gen.Inputs, dev="cuda:0"):
    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    sink = torch.from_numpy(inp.sink).to(dev) if inp.sink is not None else None
    return t(inp.q), t(inp.k), t(inp.v), sink


def run_gpu(w: Workload, q, k, v, sink, num_splits=0):
    if w.decode:
        return attn.decode(q, k, v, scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal,
                           window=w.window, n_reg=w.n_reg, sink=sink, num_splits=num_splits)
    return attn.fwd(q, k, v, scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal,
                    window=w.window, n_reg=w.n_reg, sink=sink)


def sample_rows(w: Workload, per_head: int = 4, extra: int = 256, seed: int = 0):
    """Flat row indices (n*Hq+h)*L+i: every head's first/last rows plus random rows."""
    r = np.random.default_rng(seed)
    rows = set()
    for n in range(w.N):
        for h in range(w.Hq):
            base = (n * w.Hq + h) * w.L
            for i in {0, w.L - 1, min(w.L - 1, 127), min(w.L - 1, 128), min(w.L - 1, 255), min(w.L - 1, 256)}:
                rows.add(base + i)
            for i in r.integers(0, w.L, per_head):
                rows.add(base + int(i))
    total = w.N * w.Hq * w.L
    for x in r.integers(0, total, extra):
        rows.add(int(x))
    return np.array(sorted(rows), dtype=np.int64)


def compare(w: Workload, inp: gen.Inputs, o_gpu: torch.Tensor, lse_gpu: torch.Tensor, rows=None, threads=0,
            bias=None, key_len=None):
    """Max-abs errors of O and LSE against the oracle (all rows or the given flat rows);
    bias / key_len (numpy) are passed to the oracle as the general bias."""
    if bias is None and key_len is None:
        o_ref, lse_ref = oracle.attn_workload(inp, rows=rows, threads=threads)
    else:
        o_ref, lse_ref = oracle.attn(inp.q, inp.k, inp.v, mode=w.mode, scale=w.scale, gamma=w.gamma,
                                     causal=w.causal, window=w.window, n_reg=w.n_reg, sink=inp.sink, bias=bias,
                                     key_len=key_len, rows=rows, threads=threads)
    og = o_gpu.float().cpu().numpy().astype(np.float64).reshape(-1, w.E)
    lg = lse_gpu.cpu().numpy().astype(np.float64).reshape(-1)
    o_ref = o_ref.reshape(-1, w.E)
    lse_ref = lse_ref.reshape(-1)
    if rows is not None:
        og = og[rows]
        lg = lg[rows]
    assert np.all(np.isfinite(og)), "non-finite output"
    both_ninf = np.isneginf(lg) & np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lse_ref)), "LSE -inf pattern differs"
    assert not np.any(np.isnan(lg)), "NaN LSE"
    eo = np.abs(og - o_ref)
    with np.errstate(invalid="ignore"):
        el = np.where(both_ninf, 0.0, np.abs(lg - lse_ref))
    worst = np.unravel_index(int(np.argmax(eo)), eo.shape) if eo.size else None
    return float(eo.max()) if eo.size else 0.0, float(el.max()) if el.size else 0.0, worst


def check(w: Workload, inp: gen.Inputs, o_gpu, lse_gpu, rows=None, threads=0, bias=None, key_len=None):
    eo, el, worst = compare(w, inp, o_gpu, lse_gpu, rows=rows, threads=threads, bias=bias, key_len=key_len)
    say(f"  {w.name}: max|dO|={eo:.3e} (worst row/col {worst}) max|dLSE|={el:.3e}")
    assert eo <= TOL_O[w.dtype], f"{w.name}: O error {eo:.3e} > {TOL_O[w.dtype]}"
    assert el <= TOL_LSE, f"{w.name}: LSE error {el:.3e} > {TOL_LSE}"
    return eo, el


def check_socket_heads(w: Workload, inp: gen.Inputs, top_k: int, sc_ref, sel_ref, o_ref, l_ref, og, lg, sg,
                       heads=None):
    """Check a SOCKET sparse decode head by head; returns the number of heads whose top-k is unique.

    sc_ref, sel_ref, o_ref, l_ref: the oracle's scores (fp64), selection and sparse output;
    og, lg, sg: the GPU's output, LSE and selected key indices (numpy).  heads: (n, h) pairs
    to check (default: all).  For every head the selection must be valid against the
    oracle's scores (ascending, top_k keys, every key clearly above the k-th score s_k
    chosen, every chosen key at least s_k (1 - 1e-4): fp32 against fp64 scores); where it
    is unique (no other key within that band) it must equal the oracle's.  Several
    selections are correct only when scores tie within the band; for every head, unique or
    not, the output must then be exact attention (oracle) over the keys the GPU chose,
    within the element type's O bar (2e-2 bf16, 1e-4 fp32) and 1e-3 on the LSE, and for
    unique heads the oracle's own sparse output too.
    """
    G = w.Hq // w.Hkv
    tol_o = TOL_O[w.dtype]
    unique = 0
    heads = heads if heads is not None else [(n, h) for n in range(w.N) for h in range(w.Hq)]
    for n, h in heads:
        sc = sc_ref[n, h]
        sk = np.sort(sc)[::-1][top_k - 1]
        hi, lo = sk * (1 + 1e-4), sk * (1 - 1e-4)
        chosen = np.zeros(sc.shape[0], bool)
        chosen[sg[n, h]] = True
        assert np.all(np.diff(sg[n, h]) > 0), f"head {(n, h)}: selection not ascending / repeated"
        assert chosen.sum() == top_k
        assert np.all(chosen[sc > hi]), f"head {(n, h)}: a clearly better key was left out"
        assert np.all(sc[chosen] >= lo), f"head {(n, h)}: a clearly worse key was chosen"
        if np.sum(sc >= lo) == top_k:  # the top-k set is unique
            unique += 1
            assert np.array_equal(sg[n, h], sel_ref[n, h]), f"head {(n, h)}: selection differs"
            assert np.max(np.abs(og[n, h] - o_ref[n, h])) <= tol_o
            assert abs(lg[n, h, 0] - l_ref[n, h, 0]) <= TOL_LSE
        kh = h // G
        idx = np.asarray(sg[n, h], dtype=np.int64)
        kk = np.ascontiguousarray(inp.k[n:n + 1, kh:kh + 1, idx])
        vv = np.ascontiguousarray(inp.v[n:n + 1, kh:kh + 1, idx])
        sk_h = None if inp.sink is None else np.asarray(inp.sink, dtype=np.float64)[h:h + 1]
        o_sel, l_sel = oracle.attn(np.ascontiguousarray(inp.q[n:n + 1, h:h + 1]), kk, vv, mode=w.mode,
                                   scale=w.scale, gamma=w.gamma, sink=sk_h)
        eo = float(np.max(np.abs(og[n, h] - o_sel[0, 0])))
        el = float(abs(lg[n, h, 0] - l_sel[0, 0, 0]))
        assert eo <= tol_o and el <= TOL_LSE, \
            f"head {(n, h)}: attention over the chosen keys off by {eo:.3e} / {el:.3e}"
    return unique
