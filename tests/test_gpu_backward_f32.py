"""GPU parity of the float32 backward pass (attn_bwd with dt = f32) against the
fp64 oracle's gradients.

The GPU fp32 forward produces O and LSE, the GPU fp32 backward takes them with
a seeded N(0, 1) float32 upstream gradient, and dQ, dK, dV and d sink are
compared with the oracle's exact gradients.  Bar (derived from the arithmetic:
every operand and product is fp32, relative rounding 2^-24 per operation,
accumulated over at most a few thousand terms): for each of dQ, dK, dV,
max|g - g_ref| <= 1e-4 * max|g_ref|; for d sink, |d - d_ref| <= 1e-4 *
sum_i p_sink_i |D_i| (the sum it is made of).  The cases cover both head
dimensions and score modes, GQA, sinks, windows (narrower and wider than the
tiles), register rows, rows with nothing visible, L < S and ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import say, to_device
from workloads import gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu
TOL = 1e-4


def W(name, N=1, Hq=2, Hkv=2, L=64, S_real=64, E=64, mode="dot", scale=None, gamma=0.125, causal=True, window=0,
      n_reg=0, sink=False, seed=61, k_dist="normal"):
    if scale is None:
        scale = 1.0 / np.sqrt(E)
    return Workload(name, "f32", N, Hq, Hkv, L, S_real, E, mode, float(scale), float(gamma), causal, window,
                    n_reg, sink, False, seed, k_dist)


CASES = [
    W("f32_dot_causal_e128_ragged", Hq=3, Hkv=3, L=300, S_real=300, E=128),
    W("f32_dot_noncausal_gqa_sink_L_lt_S", N=2, Hq=8, Hkv=2, L=130, S_real=190, causal=False, sink=True),
    W("f32_rbf_causal_registers_lognormal", L=257, S_real=257, mode="rbf", n_reg=4, k_dist="dir_lognormal"),
    W("f32_rbf_window_gqa_sink_e128", Hq=4, Hkv=2, L=333, S_real=333, E=128, mode="rbf", window=100, sink=True,
      gamma=0.05),
    W("f32_dot_L_gt_S_empty_rows", L=200, S_real=70),
    W("f32_dot_window_registers_sink_e128", L=400, S_real=400, E=128, window=37, n_reg=3, sink=True),
    W("f32_dot_negative_scale", N=2, L=150, S_real=150, causal=False, scale=-0.1),
    W("f32_rbf_noncausal_many_registers_e128", L=130, S_real=90, E=128, mode="rbf", n_reg=70, causal=False),
    W("f32_dot_wide_window_gqa4_e64", Hq=8, Hkv=2, L=700, S_real=700, window=300),
    W("f32_rbf_wide_window_registers_sink_e128", L=650, S_real=650, E=128, mode="rbf", window=260, n_reg=4,
      sink=True, gamma=0.05),
]


def _run(w):
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    do_np = gen.bias_f32(w.seed + 100, (w.N, w.Hq, w.L, w.E))  # seeded N(0,1) upstream gradient
    do = torch.from_numpy(do_np).to("cuda:0")
    kw = dict(scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window, n_reg=w.n_reg, sink=sink)
    o, lse = attn.fwd(q, k, v, **kw)
    dq, dk, dv, dsink = attn.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(inp.q, inp.k, inp.v, do_np, mode=w.mode, scale=w.scale, gamma=w.gamma, causal=w.causal,
                          window=w.window, n_reg=w.n_reg, sink=inp.sink)
    return (dq, dk, dv, dsink), ref, inp


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_f32(w):
    say(f"[bwd f32] {w}")
    (dq, dk, dv, dsink), ref, inp = _run(w)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert t.dtype == torch.float32
        g = t.cpu().numpy().astype(np.float64).reshape(-1, w.E)
        r = ref[name].reshape(-1, w.E)
        assert np.all(np.isfinite(g)), f"{name}: non-finite gradient"
        scale = max(np.abs(r).max(), 1e-6)
        err = np.abs(g - r).max() / scale
        say(f"  {w.name} {name}: max|err|/max|ref| = {err:.3e} (max|ref| {scale:.3e})")
        assert err <= TOL, f"{w.name} {name}: {err:.3e} > {TOL}"
    if inp.sink is not None:
        ps = np.exp(inp.sink[None, :, None] - ref["lse"])
        bound = 1e-4 * np.sum(ps * np.abs(ref["delta"]), axis=(0, 2)) + 1e-7
        d = dsink.cpu().numpy().astype(np.float64)
        say(f"  {w.name} dsink: max|err| = {np.abs(d - ref['dsink']).max():.3e} (bound {bound.min():.3e}..)")
        assert np.all(np.abs(d - ref["dsink"]) <= bound)


def test_backward_f32_deterministic():
    w = W("f32_determinism", N=2, Hq=4, Hkv=2, L=200, S_real=260, E=128, sink=True)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    do = torch.from_numpy(gen.bias_f32(w.seed + 100, (w.N, w.Hq, w.L, w.E))).to("cuda:0")
    o, lse = attn.fwd(q, k, v, causal=True, sink=sink)
    a = attn.bwd(q, k, v, o, lse, do, causal=True, sink=sink)
    b = attn.bwd(q, k, v, o, lse, do, causal=True, sink=sink)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
