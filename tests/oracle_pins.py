"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Every pin takes an oracle library handle (``lib``) and raises AssertionError if
the oracle disagrees.  test_oracle_pins.py runs them on the real oracle;
test_oracle_mutants.py runs them on copies of the oracle with planted mistakes
and requires each mistake to be caught by at least one pin.

Independent references used here: torch.nn.functional.scaled_dot_product_attention
in float64 with an explicit bottom-right boolean mask (the library routine the
SDPA page compares against, its section 1 and section 4 pitfall 3), torch.cdist
for the RBF distance (RBF digest, paragraph 2), closed forms, invariants and two
values printed on the pages (tests/golden/).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, N, Hq, Hkv, L, S, E, dtype=np.float64):
    r = _rng(seed)
    q = r.standard_normal((N, Hq, L, E)).astype(dtype)
    k = r.standard_normal((N, Hkv, S, E)).astype(dtype)
    v = r.standard_normal((N, Hkv, S, E)).astype(dtype)
    return q, k, v


def _torch_mask(L, S, causal, window):
    """Bottom-right causal / window band built from torch.tril / torch.triu (True = attend)."""
    m = torch.ones(L, S, dtype=torch.bool)
    if causal:
        m = torch.tril(m, diagonal=S - L)
    if window > 0:
        m = m & torch.triu(torch.ones(L, S, dtype=torch.bool), diagonal=S - L - window + 1)
    return m


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch"
    m = float(err.max()) if err.size else 0.0
    assert m <= tol, f"{what}: max abs err {m:.3e} > {tol:.1e}"


def _bitwise(a, b, what):
    assert np.array_equal(np.asarray(a).view(np.uint64), np.asarray(b).view(np.uint64)), f"{what}: not bitwise equal"


# --------------------------------------------------------------------------- dot mode vs library


DOT_CASES = [
    # N, Hq, Hkv, L, S, E, causal, window
    (2, 3, 3, 5, 5, 8, False, 0),
    (1, 4, 2, 7, 11, 16, True, 0),
    (2, 2, 1, 9, 9, 4, True, 0),
    (1, 2, 2, 6, 13, 8, True, 4),
    (1, 6, 3, 1, 10, 8, True, 0),
]


def pin_dot_matches_torch_sdpa(lib):
    for c, (N, Hq, Hkv, L, S, E, causal, window) in enumerate(DOT_CASES):
        q, k, v = _qkv(100 + c, N, Hq, Hkv, L, S, E)
        scale = 0.7 / math.sqrt(E)
        o, lse = oracle.attn(q, k, v, scale=scale, causal=causal, window=window, lib=lib)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        mask = _torch_mask(L, S, causal, window)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                             enable_gqa=(Hq != Hkv)).numpy()
        _close(o, ref, 1e-12, f"dot case {c} O")
        kr = tk.repeat_interleave(Hq // Hkv, dim=1)
        logits = (tq @ kr.transpose(-1, -2)) * scale
        lref = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1).numpy()
        _close(lse, lref, 1e-12, f"dot case {c} LSE")


def pin_causal_lower_right_library_mask(lib):
    """The bottom-right rule equals torch's causal_lower_right bias, named on the SDPA page."""
    from torch.nn.attention.bias import causal_lower_right
    for (L, S) in [(1, 6), (3, 5), (4, 4), (2, 9)]:
        dense = causal_lower_right(L, S)._materialize().numpy()
        mine = np.array([[oracle.visible(L, S, True, 0, 0, i, j, lib=lib) for j in range(S)] for i in range(L)])
        assert np.array_equal(dense, mine), f"visibility L={L} S={S} differs from causal_lower_right"


# --------------------------------------------------------------------------- rbf mode


RBF_CASES = [
    (1, 2, 2, 6, 6, 8, True, 0, 0),
    (2, 4, 2, 5, 9, 4, True, 0, 2),
    (1, 3, 1, 7, 7, 16, False, 0, 1),
    (1, 2, 2, 8, 12, 8, True, 3, 2),
]


def pin_rbf_matches_cdist(lib):
    gamma = 0.3
    for c, (N, Hq, Hkv, L, S, E, causal, window, n_reg) in enumerate(RBF_CASES):
        q, k, v = _qkv(200 + c, N, Hq, Hkv, L, S, E)
        o, lse = oracle.attn(q, k, v, mode="rbf", gamma=gamma, causal=causal, window=window,
                             n_reg=n_reg, lib=lib)
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
        tv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
        d2 = torch.cdist(tq, tk, compute_mode="donot_use_mm_for_euclid_dist") ** 2
        mask = torch.ones(L, S, dtype=torch.bool)
        mask[:, n_reg:] = _torch_mask(L, S - n_reg, causal, window)
        z = (-gamma * d2).masked_fill(~mask, float("-inf"))
        ref = (torch.softmax(z, dim=-1) @ tv).numpy()
        _close(o, ref, 1e-12, f"rbf case {c} O")
        _close(lse, torch.logsumexp(z, dim=-1).numpy(), 1e-11, f"rbf case {c} LSE")


def pin_rbf_tiny_loops(lib):
    """Brute force in plain Python loops on a 2-query, 3-key, E=2 problem."""
    q = np.array([[[[0.5, -1.0], [2.0, 0.25]]]])
    k = np.array([[[[1.0, 0.0], [-0.5, 0.5], [0.0, 2.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, -1.0], [0.5, 0.5]]]])
    g = 0.7
    o, lse = oracle.attn(q, k, v, mode="rbf", gamma=g, lib=lib)
    for i in range(2):
        w = []
        for j in range(3):
            d = sum((q[0, 0, i, e] - k[0, 0, j, e]) ** 2 for e in range(2))
            w.append(math.exp(-g * d))
        tot = sum(w)
        for e in range(2):
            ref = sum(w[j] * v[0, 0, j, e] for j in range(3)) / tot
            assert abs(o[0, 0, i, e] - ref) < 1e-14, "rbf tiny O"
        assert abs(lse[0, 0, i] - math.log(tot)) < 1e-14, "rbf tiny LSE"


def pin_rbf_fold_identity(lib):
    """Folded logits gamma*(2 q.k - |k|^2) give the same O; LSE differs by exactly gamma*|q|^2."""
    gamma = 0.25
    N, H, L, S, E = 1, 2, 6, 6, 8
    q, k, v = _qkv(300, N, H, H, L, S, E)
    o, lse = oracle.attn(q, k, v, mode="rbf", gamma=gamma, causal=True, lib=lib)
    zf = gamma * (2.0 * np.einsum("nhie,nhje->nhij", q, k) - np.sum(k * k, -1)[:, :, None, :])
    mask = np.tril(np.ones((L, S), bool))
    zf = np.where(mask, zf, -np.inf)
    mx = zf.max(-1, keepdims=True)
    w = np.exp(zf - mx)
    of = np.einsum("nhij,nhje->nhie", w / w.sum(-1, keepdims=True), v)
    lse_fold = (mx[..., 0] + np.log(w.sum(-1)))
    _close(o, of, 1e-12, "fold O")
    _close(lse, lse_fold - gamma * np.sum(q * q, -1), 1e-11, "fold LSE")


def pin_rbf_translation_invariance(lib):
    gamma = 0.2
    q, k, v = _qkv(310, 1, 2, 1, 5, 7, 8)
    t = _rng(311).standard_normal(8)
    o1, l1 = oracle.attn(q, k, v, mode="rbf", gamma=gamma, causal=True, lib=lib)
    o2, l2 = oracle.attn(q + t, k + t, v, mode="rbf", gamma=gamma, causal=True, lib=lib)
    _close(o1, o2, 1e-12, "rbf translation O")
    _close(l1, l2, 1e-11, "rbf translation LSE")


def pin_rbf_huge_keys_fall_to_registers(lib):
    """All real keys very far away: the output is the mean of the register values."""
    gamma = 0.125
    N, H, L, S_real, E, n_reg = 1, 2, 4, 6, 8, 3
    r = _rng(320)
    q = r.standard_normal((N, H, L, E))
    k = r.standard_normal((N, H, n_reg + S_real, E))
    k[:, :, :n_reg] = 0.0
    k[:, :, n_reg:] *= 1e3
    v = r.standard_normal((N, H, n_reg + S_real, E))
    o, _ = oracle.attn(q, k, v, mode="rbf", gamma=gamma, causal=True, n_reg=n_reg, lib=lib)
    ref = np.broadcast_to(v[:, :, None, :n_reg].mean(axis=3), o.shape)
    _close(o, ref, 1e-12, "registers absorb everything")


# --------------------------------------------------------------------------- sink


def pin_sink_minus_inf_is_no_sink(lib):
    q, k, v = _qkv(400, 1, 4, 2, 6, 9, 8)
    a = oracle.attn(q, k, v, causal=True, lib=lib)
    b = oracle.attn(q, k, v, causal=True, sink=np.full(4, -np.inf), lib=lib)
    _bitwise(a[0], b[0], "sink=-inf O")
    _bitwise(a[1], b[1], "sink=-inf LSE")


def pin_sink_closed_form(lib):
    """O_sink = O * sigmoid(LSE - s), LSE_sink = logaddexp(LSE, s)."""
    for mode, gamma in (("dot", 0.0), ("rbf", 0.2)):
        q, k, v = _qkv(410, 2, 4, 2, 6, 8, 8)
        s = _rng(411).standard_normal(4) * 2.0
        o, l = oracle.attn(q, k, v, mode=mode, gamma=gamma, causal=True, window=4, lib=lib)
        os_, ls = oracle.attn(q, k, v, mode=mode, gamma=gamma, causal=True, window=4, sink=s, lib=lib)
        sh = s[None, :, None]
        att = 1.0 / (1.0 + np.exp(sh - l))
        _close(os_, o * att[..., None], 1e-12, f"{mode} sink attenuation O")
        _close(ls, np.logaddexp(l, sh), 1e-12, f"{mode} sink LSE")


def pin_zero_sink_is_zero_token(lib):
    """Sink logit 0 in dot mode == one extra always-visible key with k = 0 and v = 0."""
    N, Hq, Hkv, L, S, E = 1, 4, 2, 5, 7, 8
    q, k, v = _qkv(420, N, Hq, Hkv, L, S, E)
    k0 = np.concatenate([np.zeros((N, Hkv, 1, E)), k], axis=2)
    v0 = np.concatenate([np.zeros((N, Hkv, 1, E)), v], axis=2)
    for causal in (False, True):
        a = oracle.attn(q, k, v, causal=causal, sink=np.zeros(Hq), lib=lib)
        b = oracle.attn(q, k0, v0, causal=causal, n_reg=1, lib=lib)
        _close(a[0], b[0], 1e-12, "zero sink O")
        _close(a[1], b[1], 1e-12, "zero sink LSE")


def pin_row_sums(lib):
    q, k, v = _qkv(430, 1, 2, 2, 6, 8, 8)
    s = np.array([0.5, -1.5])
    _, l, p = oracle.attn(q, k, v, causal=True, want_p=True, lib=lib)
    _close(p.sum(-1), np.ones_like(l), 1e-12, "row sums")
    _, l, p = oracle.attn(q, k, v, causal=True, sink=s, want_p=True, lib=lib)
    _close(p.sum(-1), 1.0 - np.exp(s[None, :, None] - l), 1e-12, "row sums with sink")


# --------------------------------------------------------------------------- masking


def _vis_matrix(L, S, causal, window, n_reg):
    m = np.zeros((L, S), bool)
    m[:, :n_reg] = True
    if S > n_reg:
        m[:, n_reg:] = _torch_mask(L, S - n_reg, causal, window).numpy()
    return m


def pin_masked_weights_exactly_zero(lib):
    for (L, S, causal, window, n_reg) in [(6, 6, True, 0, 0), (4, 9, True, 3, 2), (5, 5, False, 0, 1)]:
        q, k, v = _qkv(500, 1, 2, 2, L, S, 8)
        _, _, p = oracle.attn(q, k, v, causal=causal, window=window, n_reg=n_reg, want_p=True, lib=lib)
        vis = _vis_matrix(L, S, causal, window, n_reg)
        assert np.all(p[..., ~vis] == 0.0), "masked weight not exactly zero"
        assert np.all(p[..., vis] > 0.0), "visible weight not positive"


def pin_invisible_values_do_not_matter(lib):
    L = S = 7
    q, k, v = _qkv(510, 1, 2, 2, L, S, 8)
    v2 = v.copy()
    v2[:, :, -1] += 1000.0  # last key: visible to the last query only
    a, _ = oracle.attn(q, k, v, causal=True, lib=lib)
    b, _ = oracle.attn(q, k, v2, causal=True, lib=lib)
    _bitwise(a[:, :, :-1], b[:, :, :-1], "causal rows that cannot see the last key")
    v3 = v.copy()
    v3[:, :, 0] -= 1000.0  # first key: outside a width-3 window for queries 3..6
    a, _ = oracle.attn(q, k, v, causal=True, window=3, lib=lib)
    b, _ = oracle.attn(q, k, v3, causal=True, window=3, lib=lib)
    _bitwise(a[:, :, 3:], b[:, :, 3:], "window rows that cannot see the first key")


def pin_window_at_least_S_is_causal(lib):
    q, k, v = _qkv(520, 1, 2, 1, 6, 10, 8)
    a = oracle.attn(q, k, v, causal=True, lib=lib)
    b = oracle.attn(q, k, v, causal=True, window=10, lib=lib)
    _bitwise(a[0], b[0], "window>=S O")
    _bitwise(a[1], b[1], "window>=S LSE")


def pin_window_one_closed_form(lib):
    """window=1: each query sees only its own aligned key, O_i = v_i', LSE_i = l_i,i'."""
    L, S, E = 5, 8, 8
    q, k, v = _qkv(530, 1, 2, 2, L, S, E)
    scale = 0.3
    o, lse = oracle.attn(q, k, v, scale=scale, causal=True, window=1, lib=lib)
    off = S - L
    for i in range(L):
        _bitwise(o[:, :, i], v[:, :, i + off], f"window=1 O row {i}")
        ref = scale * np.sum(q[:, :, i] * k[:, :, i + off], -1)
        _close(lse[:, :, i], ref, 1e-13, f"window=1 LSE row {i}")


def pin_decode_alignment_golden(lib):
    with open(os.path.join(GOLDEN, "sdpa_causal_alignment_L1_S6.json")) as f:
        g = json.load(f)
    L, S = g["L"], g["S"]
    br = [oracle.visible(L, S, True, 0, 0, 0, j, lib=lib) for j in range(S)]
    assert all(br) == g["bottom_right_equals_unmasked_at_L1"], "L=1 bottom-right must see every key"
    # top-left and bottom-right coincide when L == S: the first row of the S x S rule is the printed row
    first = [oracle.visible(S, S, True, 0, 0, 0, j, lib=lib) for j in range(S)]
    assert first == g["top_left_mask"][0], "L=S causal first row differs from the printed mask"
    q, k, v = _qkv(540, 1, 2, 2, L, S, 8)
    a = oracle.attn(q, k, v, causal=True, lib=lib)
    b = oracle.attn(q, k, v, causal=False, lib=lib)
    _bitwise(a[0], b[0], "L=1 causal vs unmasked")


def pin_fully_masked_rows(lib):
    """L > S with bottom-right causal: the first L-S rows see nothing -> O = 0, LSE = -inf (or s_h)."""
    q, k, v = _qkv(550, 1, 2, 2, 4, 2, 8)
    o, l = oracle.attn(q, k, v, causal=True, lib=lib)
    assert np.all(o[:, :, :2] == 0.0) and np.all(np.isneginf(l[:, :, :2])), "empty rows"
    assert np.all(np.isfinite(o[:, :, 2:])) and np.all(np.isfinite(l[:, :, 2:])), "non-empty rows"
    s = np.array([0.3, -2.0])
    o, l = oracle.attn(q, k, v, causal=True, sink=s, lib=lib)
    assert np.all(o[:, :, :2] == 0.0), "empty rows with sink: O"
    assert np.array_equal(l[0, :, 0], s) and np.array_equal(l[0, :, 1], s), "empty rows with sink: LSE = s_h"


# --------------------------------------------------------------------------- uniform weights


def pin_equal_logits_give_uniform_average(lib):
    N, Hq, Hkv, L, S, E = 1, 4, 2, 6, 9, 8
    _, k, v = _qkv(600, N, Hq, Hkv, L, S, E)
    q = np.zeros((N, Hq, L, E))
    o, lse = oracle.attn(q, k, v, causal=True, window=5, n_reg=1, lib=lib)
    vis = _vis_matrix(L, S, True, 5, 1)
    for h in range(Hq):
        kh = h // (Hq // Hkv)
        for i in range(L):
            sel = v[0, kh, vis[i]]
            _close(o[0, h, i], sel.mean(0), 1e-14, "uniform average")
            _close(lse[0, h, i], math.log(sel.shape[0]), 1e-14, "LSE = ln n_visible")


def pin_uniform_entropy_golden(lib):
    with open(os.path.join(GOLDEN, "attention_uniform_entropy_n24.json")) as f:
        g = json.load(f)
    n = g["n"]
    _, k, v = _qkv(610, 1, 1, 1, 3, n, 4)
    q = np.zeros((1, 1, 3, 4))
    _, _, p = oracle.attn(q, k, v, want_p=True, lib=lib)
    ent = -np.sum(p * np.log(p), -1).mean()
    assert round(float(ent), g["decimals"]) == g["mean_row_entropy"], f"entropy {ent}"


# --------------------------------------------------------------------------- invariances


def pin_shift_invariance(lib):
    """Adding c_i to every logit of row i (via an extra coordinate) keeps O, shifts LSE by c_i."""
    N, H, L, S, E = 1, 2, 5, 7, 8
    q, k, v = _qkv(700, N, H, H, L, S, E)
    scale = 0.4
    c = _rng(701).standard_normal((N, H, L)) * 3.0
    q2 = np.concatenate([q, (c / scale)[..., None]], -1)
    k2 = np.concatenate([k, np.ones((N, H, S, 1))], -1)
    o1, l1 = oracle.attn(q, k, v, scale=scale, causal=True, lib=lib)
    v2 = v  # E_v stays 8: pad V to the new head size and drop the pad afterwards
    v2p = np.concatenate([v2, np.zeros((N, H, S, 1))], -1)
    o2, l2 = oracle.attn(q2, k2, v2p, scale=scale, causal=True, lib=lib)
    _close(o2[..., :E], o1, 1e-12, "shifted O")
    _close(l2, l1 + c, 1e-12, "shifted LSE")


def pin_permutation_equivariance(lib):
    N, H, L, S, E = 1, 2, 6, 8, 8
    q, k, v = _qkv(710, N, H, H, L, S, E)
    o, l = oracle.attn(q, k, v, lib=lib)
    pq = _rng(711).permutation(L)
    o2, l2 = oracle.attn(q[:, :, pq], k, v, lib=lib)
    _bitwise(o2, o[:, :, pq], "query permutation O")
    _bitwise(l2, l[:, :, pq], "query permutation LSE")
    pk = _rng(712).permutation(S)
    o3, l3 = oracle.attn(q, k[:, :, pk], v[:, :, pk], lib=lib)
    _close(o3, o, 1e-12, "key permutation O")
    _close(l3, l, 1e-12, "key permutation LSE")


def pin_gqa_equals_repeat(lib):
    N, Hq, Hkv, L, S, E = 2, 6, 2, 5, 8, 8
    q, k, v = _qkv(720, N, Hq, Hkv, L, S, E)
    G = Hq // Hkv
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    for mode in ("dot", "rbf"):
        a = oracle.attn(q, k, v, mode=mode, gamma=0.2, causal=True, lib=lib)
        b = oracle.attn(q, kr, vr, mode=mode, gamma=0.2, causal=True, lib=lib)
        _bitwise(a[0], b[0], f"{mode} GQA O")
        _bitwise(a[1], b[1], f"{mode} GQA LSE")


def pin_convex_hull(lib):
    q, k, v = _qkv(730, 1, 2, 2, 6, 6, 8)
    o, _ = oracle.attn(q, k, v, causal=True, lib=lib)
    for i in range(6):
        lo = v[:, :, :i + 1].min(2)
        hi = v[:, :, :i + 1].max(2)
        assert np.all(o[:, :, i] >= lo - 1e-12) and np.all(o[:, :, i] <= hi + 1e-12), "outside hull"
    o, _ = oracle.attn(q, k, v, causal=True, sink=np.array([1.0, 2.0]), lib=lib)
    for i in range(6):
        lo = np.minimum(v[:, :, :i + 1].min(2), 0.0)
        hi = np.maximum(v[:, :, :i + 1].max(2), 0.0)
        assert np.all(o[:, :, i] >= lo - 1e-12) and np.all(o[:, :, i] <= hi + 1e-12), "outside hull with 0"


# --------------------------------------------------------------------------- input types, row sampling


def pin_bf16_widening(lib):
    r = _rng(800)
    bits = [(r.standard_normal(s).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            for s in ((1, 2, 5, 8), (1, 1, 7, 8), (1, 1, 7, 8))]
    wide = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy() for b in bits]
    a = oracle.attn(*bits, causal=True, lib=lib)
    b = oracle.attn(*wide, causal=True, lib=lib)
    _bitwise(a[0], b[0], "bf16 O")
    _bitwise(a[1], b[1], "bf16 LSE")


def pin_f32_widening(lib):
    q, k, v = _qkv(810, 1, 2, 1, 5, 7, 8, dtype=np.float32)
    a = oracle.attn(q, k, v, mode="rbf", gamma=0.3, causal=True, lib=lib)
    b = oracle.attn(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), mode="rbf",
                    gamma=0.3, causal=True, lib=lib)
    _bitwise(a[0], b[0], "f32 O")
    _bitwise(a[1], b[1], "f32 LSE")


def pin_row_sampling(lib):
    q, k, v = _qkv(820, 2, 4, 2, 6, 9, 8)
    s = np.array([0.1, -0.2, 0.3, 1.0])
    full = oracle.attn(q, k, v, causal=True, window=4, sink=s, lib=lib)
    rows = [0, 5, 13, 47, 22]
    part = oracle.attn(q, k, v, causal=True, window=4, sink=s, rows=rows, lib=lib)
    _bitwise(part[0], full[0].reshape(-1, 8)[rows], "sampled O")
    _bitwise(part[1], full[1].reshape(-1)[rows], "sampled LSE")


def pin_float_bias_matches_sdpa_mask(lib):
    # SDPA page section 1: softmax(QK^T*scale + B) V with a float B (torch's attn_mask)
    q, k, v = _qkv(61, 2, 3, 3, 6, 9, 8)
    b = _rng(62).standard_normal((2, 1, 6, 9)).astype(np.float32)
    b[1, 0, 2, [1, 4]] = -np.inf
    o, _ = oracle.attn(q, k, v, scale=0.3, bias=b, lib=lib)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(b.astype(np.float64)), scale=0.3)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12


def pin_bool_mask_true_means_attend(lib):
    # SDPA page section 4: in attn_mask, True = the pair takes part
    q, k, v = _qkv(63, 1, 2, 2, 5, 7, 8)
    m = _rng(64).random((1, 2, 5, 7)) < 0.5
    m[..., 3] = True
    o, _ = oracle.attn(q, k, v, bias=m, lib=lib)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(m))
    assert np.max(np.abs(o - ref.numpy())) < 1e-12


def pin_key_padding_equals_slicing(lib):
    # padded keys take no part: same as cutting K/V after the valid ones
    q, k, v = _qkv(65, 2, 2, 2, 4, 10, 8)
    o, lse = oracle.attn(q, k, v, key_len=[6, 10], lib=lib)
    o1, l1 = oracle.attn(q[:1], k[:1, :, :6], v[:1, :, :6], lib=lib)
    assert np.max(np.abs(o[:1] - o1)) < 1e-12 and np.max(np.abs(lse[:1] - l1)) < 1e-12


# ----------------------------------------------------------------------------- backward


def _visible_mask(L, S, causal, window, n_reg):
    m = np.zeros((L, S), bool)
    for i in range(L):
        for j in range(S):
            if j < n_reg:
                m[i, j] = True
                continue
            r, ip = j - n_reg, i + (S - n_reg - L)
            m[i, j] = (not causal or r <= ip) and (window <= 0 or ip - r < window)
    return m


def pin_bwd_dot_matches_sdpa_autograd(lib):
    # the gradient formulas against automatic differentiation of the library routine
    q, k, v = _qkv(71, 2, 4, 2, 6, 9, 8)
    do = _rng(72).standard_normal(q.shape)
    g = oracle.attn_bwd(q, k, v, do, scale=0.3, causal=True, lib=lib)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    m = torch.from_numpy(_visible_mask(6, 9, True, 0, 0))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=0.3, enable_gqa=True)
    o.backward(torch.from_numpy(do))
    for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
        assert np.max(np.abs(g[name] - t.grad.numpy())) < 1e-12, name


def pin_bwd_rbf_matches_cdist_autograd(lib):
    q, k, v = _qkv(73, 1, 2, 2, 5, 8, 6)
    do = _rng(74).standard_normal(q.shape)
    g = oracle.attn_bwd(q, k, v, do, mode="rbf", gamma=0.2, causal=True, window=3, n_reg=2, lib=lib)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    z = -0.2 * torch.cdist(qt, kt) ** 2
    z = z.masked_fill(~torch.from_numpy(_visible_mask(5, 8, True, 3, 2)), float("-inf"))
    o = torch.softmax(z, -1) @ vt
    o.backward(torch.from_numpy(do))
    for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
        assert np.max(np.abs(g[name] - t.grad.numpy())) < 1e-10, name


def pin_bwd_finite_differences_with_sink(lib):
    # central differences of L = sum(dO * O) in fp64, every input and the sink
    q, k, v = _qkv(75, 1, 4, 2, 4, 6, 3)
    do = _rng(76).standard_normal(q.shape)
    sink = _rng(77).standard_normal(4)
    kw = dict(mode="rbf", gamma=0.3, causal=True, window=3, n_reg=1)
    g = oracle.attn_bwd(q, k, v, do, sink=sink, lib=lib, **kw)

    def loss(q_, k_, v_, s_):
        o, _ = oracle.attn(q_, k_, v_, sink=s_, lib=lib, **kw)
        return float(np.sum(o * do))
    h = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            args1 = [q, k, v, sink]
            args2 = [q, k, v, sink]
            pos = {"dq": 0, "dk": 1, "dv": 2}[name]
            args1[pos], args2[pos] = a1, a2
            fd = (loss(*args1) - loss(*args2)) / (2 * h)
            assert abs(fd - g[name][idx]) < 1e-6, (name, idx, fd, g[name][idx])
    for hh in range(4):
        s1, s2 = sink.copy(), sink.copy()
        s1[hh] += h
        s2[hh] -= h
        fd = (loss(q, k, v, s1) - loss(q, k, v, s2)) / (2 * h)
        assert abs(fd - g["dsink"][hh]) < 1e-6


def pin_bwd_row_subsets_and_delta(lib):
    q, k, v = _qkv(78, 2, 2, 1, 5, 7, 4)
    do = _rng(79).standard_normal(q.shape)
    full = oracle.attn_bwd(q, k, v, do, causal=True, n_reg=1, lib=lib)
    qr, kr = [3, 7, 19], [0, 5, 13]
    part = oracle.attn_bwd(q, k, v, do, causal=True, n_reg=1, qrows=qr, krows=kr, lib=lib)
    assert np.array_equal(part["dq"], full["dq"].reshape(-1, 4)[qr])
    assert np.array_equal(part["dk"], full["dk"].reshape(-1, 4)[kr])
    assert np.array_equal(part["dv"], full["dv"].reshape(-1, 4)[kr])
    o, lse = oracle.attn(q, k, v, causal=True, n_reg=1, lib=lib)
    assert np.max(np.abs(full["delta"] - np.sum(o * do, -1))) < 1e-12
    assert np.max(np.abs(full["lse"] - lse)) < 1e-12


# ----------------------------------------------------------------------------- SOCKET


def pin_socket_soft_assignment_is_product_of_sigmoids(lib):
    # softmax over the 2^bits sign patterns of sum_b s_b y_b / tau factorises into
    # prod_b sigmoid(2 s_b y_b / tau): one key per bucket, unit value norm, one table
    bits, E, tau = 4, 8, 0.7
    r = _rng(81)
    proj = r.standard_normal((bits, E)).astype(np.float32)
    q = r.standard_normal(E)
    codes = np.arange(1 << bits, dtype=np.uint8)[:, None]
    sc = oracle.socket_scores(q, proj, codes, np.ones(1 << bits), 1, bits, tau, lib=lib)
    y = proj.astype(np.float64) @ q
    for c in range(1 << bits):
        s_ = np.array([1.0 if (c >> b) & 1 else -1.0 for b in range(bits)])
        ref = np.prod(1.0 / (1.0 + np.exp(-2.0 * s_ * y / tau)))
        assert abs(sc[c] - ref) < 1e-12


def pin_socket_low_temperature_is_hard_collision_count(lib):
    # tau -> 0: all mass on the query's own sign pattern; a key scores |v| * (tables it collides in)
    tables, bits, E = 5, 3, 8
    r = _rng(82)
    proj = r.standard_normal((tables * bits, E)).astype(np.float32)
    q = r.standard_normal(E)
    qcode = [sum(1 << b for b in range(bits) if float(proj[t * bits + b].astype(np.float64) @ q) > 0)
             for t in range(tables)]
    buckets = r.integers(0, 1 << bits, size=(40, tables)).astype(np.uint8)
    buckets[0] = qcode
    vn = r.random(40) + 0.5
    sc = oracle.socket_scores(q, proj, buckets, vn, tables, bits, 1e-4, lib=lib)
    hard = vn * np.sum(buckets == np.array(qcode, dtype=np.uint8)[None, :], axis=1)
    assert np.max(np.abs(sc - hard)) < 1e-9


def pin_socket_hash_is_random_hyperplane_signs(lib):
    # bit b of table t is sign(w_tb . k) (checked where |w.k| is clear of rounding), norms are |v|
    tables, bits, E = 4, 6, 16
    r = _rng(83)
    proj = r.standard_normal((tables * bits, E)).astype(np.float32)
    k = r.standard_normal((1, 1, 64, E)).astype(np.float32)
    v = r.standard_normal((1, 1, 64, E)).astype(np.float32)
    b, vn = oracle.socket_hash(k, v, proj, tables, bits, lib=lib)
    x = k[0, 0].astype(np.float64) @ proj.astype(np.float64).T  # (64, tables*bits)
    for j in range(64):
        for t in range(tables):
            for bb in range(bits):
                xv = x[j, t * bits + bb]
                if abs(xv) > 1e-4:
                    assert ((int(b[0, 0, j, t]) >> bb) & 1) == (1 if xv > 0 else 0)
    assert np.max(np.abs(vn[0, 0] - np.linalg.norm(v[0, 0].astype(np.float64), axis=1))) < 1e-12


def pin_socket_collision_rate_follows_angle(lib):
    # random hyperplanes: P(same bit) = 1 - angle/pi (the angular kernel the page's theory builds on)
    E, nproj = 16, 8192
    r = _rng(84)
    proj = r.standard_normal((nproj, E)).astype(np.float32)
    a = r.standard_normal(E)
    c = r.standard_normal(E)
    c = c - (c @ a) / (a @ a) * a
    b_ = a / np.linalg.norm(a) * np.cos(1.0) + c / np.linalg.norm(c) * np.sin(1.0)  # angle 1 rad to a
    keys = np.stack([a, b_])[None, None].astype(np.float32)
    codes, _ = oracle.socket_hash(keys, keys, proj, nproj, 1, lib=lib)
    same = np.mean(codes[0, 0, 0] == codes[0, 0, 1])
    expect = 1.0 - 1.0 / np.pi
    assert abs(same - expect) < 4 * np.sqrt(expect * (1 - expect) / nproj)


def pin_socket_full_budget_is_dense_attention(lib):
    # top_k = S selects every key: the sparse decode is the dense decode
    q, k, v = _qkv(85, 1, 4, 2, 1, 30, 8)
    proj = _rng(86).standard_normal((2 * 3, 8)).astype(np.float32)
    b, vn = oracle.socket_hash(k, v, proj, 2, 3, lib=lib)
    sink = _rng(87).standard_normal(4)
    o, lse, sel, _ = oracle.socket_decode(q, k, v, proj, b, vn, tables=2, bits=3, tau=0.5, top_k=30, sink=sink,
                                          lib=lib)
    o2, l2 = oracle.attn(q, k, v, sink=sink, lib=lib)
    assert np.all(sel == np.arange(30)) and np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - l2)) < 1e-12


def pin_socket_selection_is_top_k_by_score(lib):
    q, k, v = _qkv(88, 1, 2, 1, 1, 200, 8)
    proj = _rng(89).standard_normal((4 * 4, 8)).astype(np.float32)
    b, vn = oracle.socket_hash(k, v, proj, 4, 4, lib=lib)
    _, _, sel, sc = oracle.socket_decode(q, k, v, proj, b, vn, tables=4, bits=4, tau=0.3, top_k=20, lib=lib)
    for h in range(2):
        s = sc[0, h]
        chosen = np.zeros(200, bool)
        chosen[sel[0, h]] = True
        assert chosen.sum() == 20 and s[chosen].min() >= s[~chosen].max()


def pin_socket_selection_ties_to_lower_index(lib):
    # Method step 4 asks for a deterministic top-k; the reading taken is: higher score first,
    # equal scores by lower key index.  (1) A hand-worked case whose ties straddle the cut:
    # scores 5 5 | 3 3 3 3 | 1 at keys 0,6 | 1,2,3,5 | 4, top 4 -> keys 0, 6, then 1, 2.
    sel = oracle.socket_select(np.array([5.0, 3.0, 3.0, 3.0, 1.0, 3.0, 5.0]), 4, lib=lib)
    assert sel.tolist() == [0, 1, 2, 6]
    # every key tied: the first top_k keys
    assert oracle.socket_select(np.full(9, 2.5), 3, lib=lib).tolist() == [0, 1, 2]
    assert oracle.socket_select(np.array([1.0, 2.0]), 0, lib=lib).tolist() == []
    # (2) Brute force over every subset on tiny inputs with many ties: the chosen set holds
    # the top_k largest scores (as a multiset), and of all such sets it is the one whose
    # ascending index list is lexicographically smallest.
    import itertools
    r = _rng(90)
    for trial in range(60):
        S = int(r.integers(1, 10))
        k = int(r.integers(0, S + 1))
        sc = r.integers(0, 3, size=S).astype(np.float64)
        best = None
        for comb in itertools.combinations(range(S), k):
            key = (sorted((-sc[list(comb)]).tolist()), list(comb))
            if best is None or key < best:
                best = key
        assert oracle.socket_select(sc, k, lib=lib).tolist() == best[1], (sc, k)


def _round_f32_exact(x):
    """x (a Fraction) rounded to the nearest float32, ties to even (normal range only)."""
    from fractions import Fraction
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e < 128
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return (fl * quantum) if x > 0 else -(fl * quantum)


def _f32_chain_sign(k, w, order, fused):
    """Sign bit (x > 0) of a float32 dot product accumulated over `order` with exact
    rational arithmetic and one IEEE rounding per step (a fused multiply-add, or a
    rounded product then a rounded sum)."""
    from fractions import Fraction
    x = Fraction(0)
    for e in order:
        prod = Fraction(float(k[e])) * Fraction(float(w[e]))
        if fused:
            x = _round_f32_exact(prod + x)
        else:
            x = _round_f32_exact(_round_f32_exact(prod) + x)
    return 1 if x > 0 else 0


def pin_socket_hash_fp32_fma_in_element_order(lib):
    # The bucket bit is decided in float32 (reading of method step 1: the precision that
    # makes the integer decision).  Keys are built so that their projection nearly cancels
    # (the last element undoes the others to float32 precision); there the sign depends on
    # the rounding order, and the oracle must follow a fused multiply-add per element in
    # element order, modelled here with exact rational arithmetic.
    E, nkeys = 8, 400
    r = _rng(91)
    w = r.standard_normal(E).astype(np.float32)
    keys = r.standard_normal((nkeys, E)).astype(np.float32)
    head = keys[:, :E - 1].astype(np.float64) @ w[:E - 1].astype(np.float64)
    keys[:, E - 1] = (-head / float(w[E - 1])).astype(np.float32)
    codes, _ = oracle.socket_hash(keys[None, None], keys[None, None], w[None, :], 1, 1, lib=lib)
    fwd = list(range(E))
    want = np.array([_f32_chain_sign(keys[j], w, fwd, True) for j in range(nkeys)])
    got = codes[0, 0, :, 0].astype(np.int64)
    assert np.array_equal(got, want)
    # the construction really separates the conventions: element order and fusion both matter
    rev = np.array([_f32_chain_sign(keys[j], w, fwd[::-1], True) for j in range(nkeys)])
    unf = np.array([_f32_chain_sign(keys[j], w, fwd, False) for j in range(nkeys)])
    assert np.sum(rev != want) >= 10 and np.sum(unf != want) >= 10


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
