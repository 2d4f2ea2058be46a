"""GPU parity of the backward pass (attn_bwd through the C ABI) against the
fp64 oracle's gradients.

The GPU forward produces O and LSE (as in training), the GPU backward takes
them with a seeded upstream gradient, and dQ, dK, dV and d sink are compared
with the oracle's exact gradients (computed from the inputs alone).  Bar
(derived from the arithmetic: bf16 operands P and dS and bf16 outputs carry a
relative rounding of 2^-9 each, accumulation is fp32): for each of dQ, dK, dV,
max|g - g_ref| <= 2e-2 * max|g_ref|; for d sink, |d - d_ref| <= 1e-2 *
sum_i p_sink_i |D_i| (the sum it is made of).  Small shapes cover every flag
with ragged tails; the headline shape is checked on sampled rows and keys.
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import say, to_device
from workloads import configs, gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu
TOL = 2e-2


def W(name, N=1, Hq=2, Hkv=2, L=64, S_real=64, E=64, mode="dot", scale=None, gamma=0.125, causal=True, window=0,
      n_reg=0, sink=False, seed=41, k_dist="normal"):
    if scale is None:
        scale = 1.0 / np.sqrt(E)
    return Workload(name, "bf16", N, Hq, Hkv, L, S_real, E, mode, float(scale), float(gamma), causal, window,
                    n_reg, sink, False, seed, k_dist)


CASES = [
    W("dot_causal_e128_ragged", Hq=3, Hkv=3, L=300, S_real=300, E=128),
    W("dot_noncausal_gqa_sink_L_lt_S", N=2, Hq=8, Hkv=2, L=130, S_real=190, causal=False, sink=True),
    W("rbf_causal_registers_lognormal", L=257, S_real=257, mode="rbf", n_reg=4, k_dist="dir_lognormal"),
    W("rbf_window_gqa_sink_e128", Hq=4, Hkv=2, L=333, S_real=333, E=128, mode="rbf", window=100, sink=True,
      gamma=0.05),
    W("dot_L_gt_S_empty_rows", L=200, S_real=70),
    W("dot_window_registers_sink_e128", L=400, S_real=400, E=128, window=37, n_reg=3, sink=True),
    W("dot_negative_scale", N=2, L=150, S_real=150, causal=False, scale=-0.1),
    W("rbf_noncausal_many_registers_e128", L=130, S_real=90, E=128, mode="rbf", n_reg=70, causal=False),
    # windows wider than the tiles: query and key tiles seen whole by a whole
    # workgroup (no visibility code) sit between masked ones on both sides
    W("dot_wide_window_e64", L=700, S_real=700, window=300),
    W("rbf_wide_window_registers_sink_e128", L=650, S_real=650, E=128, mode="rbf", window=260, n_reg=4,
      sink=True, gamma=0.05),
]


def _upstream(w):
    g = gen.bias_f32(w.seed + 100, (w.N, w.Hq, w.L, w.E))  # seeded N(0,1) upstream gradient
    return gen.bf16_bits_from_f32(g)


def _run(w, qrows=None, krows=None):
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    do_bits = _upstream(w)
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    kw = dict(scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window, n_reg=w.n_reg, sink=sink)
    o, lse = attn.fwd(q, k, v, **kw)
    dq, dk, dv, dsink = attn.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(inp.q, inp.k, inp.v, do_bits, mode=w.mode, scale=w.scale, gamma=w.gamma, causal=w.causal,
                          window=w.window, n_reg=w.n_reg, sink=inp.sink, qrows=qrows, krows=krows)
    return (dq, dk, dv, dsink), ref, inp


def _check(w, got, ref, inp, qrows=None, krows=None):
    dq, dk, dv, dsink = got
    for name, t, rows in (("dq", dq, qrows), ("dk", dk, krows), ("dv", dv, krows)):
        g = t.float().cpu().numpy().astype(np.float64).reshape(-1, w.E)
        if rows is not None:
            g = g[rows]
        r = ref[name].reshape(-1, w.E)
        assert np.all(np.isfinite(g)), f"{name}: non-finite gradient"
        scale = max(np.abs(r).max(), 1e-6)
        err = np.abs(g - r).max() / scale
        say(f"  {w.name} {name}: max|err|/max|ref| = {err:.3e} (max|ref| {scale:.3e})")
        assert err <= TOL, f"{w.name} {name}: {err:.3e} > {TOL}"
    if inp.sink is not None:
        ps = np.exp(inp.sink[None, :, None] - ref["lse"])
        bound = 1e-2 * np.sum(ps * np.abs(ref["delta"]), axis=(0, 2)) + 1e-6
        d = dsink.cpu().numpy().astype(np.float64)
        say(f"  {w.name} dsink: max|err| = {np.abs(d - ref['dsink']).max():.3e} (bound {bound.min():.3e}..)")
        assert np.all(np.abs(d - ref["dsink"]) <= bound)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_small(w):
    say(f"[bwd] {w}")
    got, ref, inp = _run(w)
    _check(w, got, ref, inp)


def test_backward_deterministic():
    w = W("determinism", N=2, Hq=4, Hkv=2, L=200, S_real=260, E=128, sink=True)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    do = torch.from_numpy(_upstream(w).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    o, lse = attn.fwd(q, k, v, causal=True, sink=sink)
    a = attn.bwd(q, k, v, o, lse, do, causal=True, sink=sink)
    b = attn.bwd(q, k, v, o, lse, do, causal=True, sink=sink)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def _sample(total, n, seed):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, total - 1], r.integers(0, total, n)]))


def test_backward_full_c2_sampled():
    w = configs.C2
    say(f"[bwd full] {w.name}")
    qrows = _sample(w.N * w.Hq * w.L, 192, 1)
    krows = _sample(w.N * w.Hkv * w.S, 192, 2)
    got, ref, inp = _run(w, qrows=qrows, krows=krows)
    _check(w, got, ref, inp, qrows=qrows, krows=krows)


def test_backward_full_c3_sampled():
    # RBF, 4 register tokens, magnitude-skewed keys, E = 64, at full size: the
    # dQ rows and dK/dV keys sampled across every head.
    w = configs.C3
    say(f"[bwd full] {w.name}")
    qrows = _sample(w.N * w.Hq * w.L, 192, 3)
    krows = _sample(w.N * w.Hkv * w.S, 192, 4)
    got, ref, inp = _run(w, qrows=qrows, krows=krows)
    _check(w, got, ref, inp, qrows=qrows, krows=krows)
