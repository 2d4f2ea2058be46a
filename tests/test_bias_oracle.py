"""Pins of the general-bias part of the oracle (CPU only).

The SDPA page (section 1) defines Attention(Q,K,V) = softmax(QK^T/sqrt(E) + B) V
with B an L x S matrix, and section 4 fixes the boolean convention (True =
the pair is used) and the AND-combination of padding and causal masks.  The
oracle's bias path is pinned to: the library routine the page describes
(torch's scaled_dot_product_attention in float64 on the CPU, float and boolean
attn_mask), the causal rule expressed as a mask, key padding expressed as
slicing, exact identities (zero bias, all-true mask, -inf vs False, row
shifts), and a brute-force softmax on tiny inputs.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_float_bias_matches_sdpa_float_mask():
    N, H, L, S, E = 2, 3, 7, 9, 16
    q, k, v = rnd(1, N, H, L, E), rnd(2, N, H, S, E), rnd(3, N, H, S, E)
    b = rnd(4, N, H, L, S).astype(np.float32)
    b[0, 1, 2, [0, 3, 5]] = -np.inf
    o, lse = oracle.attn(q, k, v, bias=b)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(b.astype(np.float64)))
    assert np.max(np.abs(o - ref.numpy())) < 1e-12


def test_bool_mask_matches_sdpa_bool_mask_true_means_attend():
    N, H, L, S, E = 1, 2, 6, 8, 8
    q, k, v = rnd(5, N, H, L, E), rnd(6, N, H, S, E), rnd(7, N, H, S, E)
    m = np.random.default_rng(8).random((N, 1, L, S)) < 0.6
    m[..., 0] = True  # no fully masked row here (covered below)
    o, _ = oracle.attn(q, k, v, bias=m)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(m))
    assert np.max(np.abs(o - ref.numpy())) < 1e-12


def test_lower_right_causal_mask_equals_causal_rule():
    N, H, L, S, E = 2, 2, 5, 11, 8
    q, k, v = rnd(9, N, H, L, E), rnd(10, N, H, S, E), rnd(11, N, H, S, E)
    i = np.arange(L)[:, None]
    j = np.arange(S)[None, :]
    m = (j <= i + (S - L))[None, None]
    o1, l1 = oracle.attn(q, k, v, bias=m)
    o2, l2 = oracle.attn(q, k, v, causal=True)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_identities_zero_bias_all_true_and_neg_inf():
    N, H, L, S, E = 2, 4, 6, 10, 8
    q, k, v = rnd(12, N, H, L, E), rnd(13, N, 2, S, E), rnd(14, N, 2, S, E)
    kw = dict(causal=True, window=4, n_reg=2, sink=rnd(15, H))
    o0, l0 = oracle.attn(q, k, v, **kw)
    o1, l1 = oracle.attn(q, k, v, bias=np.zeros((1, 1, L, S), np.float32), **kw)
    o2, l2 = oracle.attn(q, k, v, bias=np.ones((N, H, L, S), bool), **kw)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    assert np.array_equal(o0, o2) and np.array_equal(l0, l2)
    m = np.random.default_rng(16).random((N, 1, L, S)) < 0.5
    b = np.where(m, 0.0, -np.inf).astype(np.float32)
    o3, l3 = oracle.attn(q, k, v, bias=m, **kw)
    o4, l4 = oracle.attn(q, k, v, bias=b, **kw)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


def test_row_constant_bias_shifts_lse_only():
    N, H, L, S, E = 1, 2, 4, 7, 8
    q, k, v = rnd(17, N, H, L, E), rnd(18, N, H, S, E), rnd(19, N, H, S, E)
    c = rnd(20, N, H, L, 1)
    b = np.broadcast_to(c, (N, H, L, S)).astype(np.float32)
    o0, l0 = oracle.attn(q, k, v)
    o1, l1 = oracle.attn(q, k, v, bias=np.ascontiguousarray(b))
    assert np.max(np.abs(o0 - o1)) < 1e-12
    assert np.max(np.abs((l1 - l0) - c[..., 0].astype(np.float32))) < 1e-12


def test_key_padding_equals_slicing_and_keeps_registers():
    N, H, L, S, E, n_reg = 3, 2, 5, 12, 8, 2
    q, k, v = rnd(21, N, H, L, E), rnd(22, N, H, S, E), rnd(23, N, H, S, E)
    kl = [10, 4, 0]
    o, lse = oracle.attn(q, k, v, n_reg=n_reg, key_len=kl)
    for n in range(N):
        cut = n_reg + kl[n]
        o_s, l_s = oracle.attn(q[n:n + 1], k[n:n + 1, :, :cut], v[n:n + 1, :, :cut], n_reg=n_reg)
        assert np.max(np.abs(o[n] - o_s[0])) < 1e-12 and np.max(np.abs(lse[n] - l_s[0])) < 1e-12


def test_fully_masked_rows_give_zero_and_neg_inf_or_sink():
    N, H, L, S, E = 1, 2, 3, 5, 4
    q, k, v = rnd(24, N, H, L, E), rnd(25, N, H, S, E), rnd(26, N, H, S, E)
    m = np.ones((1, 1, L, S), bool)
    m[0, 0, 1] = False
    o, lse = oracle.attn(q, k, v, bias=m)
    assert np.all(o[:, :, 1] == 0) and np.all(np.isneginf(lse[:, :, 1]))
    s = np.array([0.3, -1.0])
    o, lse = oracle.attn(q, k, v, bias=m, sink=s)
    assert np.all(o[:, :, 1] == 0) and np.allclose(lse[0, :, 1], s)


def test_brute_force_softmax_with_bias_and_sink():
    L, S, E = 3, 6, 5
    q, k, v = rnd(27, 1, 1, L, E), rnd(28, 1, 1, S, E), rnd(29, 1, 1, S, E)
    b = rnd(30, 1, 1, L, S).astype(np.float32)
    s = np.array([0.7])
    o, lse = oracle.attn(q, k, v, scale=0.4, bias=b, sink=s, causal=True)
    for i in range(L):
        z = [0.4 * float(q[0, 0, i] @ k[0, 0, j]) + float(b[0, 0, i, j]) for j in range(S) if j <= i + S - L]
        z = np.array(z)
        den = np.exp(z).sum() + np.exp(0.7)
        ref = (np.exp(z)[:, None] * v[0, 0, :len(z)]).sum(0) / den
        assert np.max(np.abs(o[0, 0, i] - ref)) < 1e-12
        assert abs(lse[0, 0, i] - np.log(den)) < 1e-12


def test_broadcast_strides():
    assert oracle.bias_strides(np.zeros((1, 1, 3, 4)), 2, 5, 3, 4) == (0, 0)
    assert oracle.bias_strides(np.zeros((2, 1, 3, 4)), 2, 5, 3, 4) == (12, 0)
    assert oracle.bias_strides(np.zeros((1, 5, 3, 4)), 2, 5, 3, 4) == (0, 12)
    assert oracle.bias_strides(np.zeros((2, 5, 3, 4)), 2, 5, 3, 4) == (60, 12)
    with pytest.raises(ValueError):
        oracle.bias_strides(np.zeros((3, 1, 3, 4)), 2, 5, 3, 4)
