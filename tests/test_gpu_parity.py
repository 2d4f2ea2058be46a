"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Small shapes cover every flag combination with ragged tails (L and S not
multiples of the tiles), L < S, L > S (rows with nothing visible), GQA, more
register rows than one key tile, and forced split counts for decode.  The five
workload configurations run at full size; where the oracle would need minutes,
it is evaluated on sampled rows (every head's first and last rows plus random
ones).  Bar: max-abs error 2e-2 on bf16 outputs, 1e-4 on fp32 outputs, 1e-3 on
the row LSE.
"""
import numpy as np
import pytest
import torch

import softmax_attention_attn_amd as attn
from gpu_util import check, run_gpu, sample_rows, say, to_device
from workloads import configs, gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu


def W(name, dtype="bf16", N=1, Hq=2, Hkv=2, L=64, S_real=64, E=64, mode="dot", scale=None, gamma=0.125,
      causal=True, window=0, n_reg=0, sink=False, decode=False, seed=11, k_dist="normal"):
    if scale is None:
        scale = 1.0 / np.sqrt(E)
    return Workload(name, dtype, N, Hq, Hkv, L, S_real, E, mode, float(scale), float(gamma), causal, window,
                    n_reg, sink, decode, seed, k_dist)


PREFILL_CASES = [
    W("dot_noncausal_mha", N=2, L=150, S_real=150, causal=False),
    W("dot_causal_e128_ragged", Hq=3, Hkv=3, L=300, S_real=300, E=128),
    W("dot_causal_L_lt_S", L=100, S_real=333, E=128),
    W("dot_causal_L_gt_S_empty_rows", L=200, S_real=70),
    W("dot_gqa_causal", Hq=8, Hkv=2, L=257, S_real=257),
    W("dot_window_sink", L=400, S_real=400, window=37, sink=True),
    W("dot_window_gqa_sink_e128", Hq=6, Hkv=3, L=520, S_real=520, E=128, window=128, sink=True),
    W("dot_sink_noncausal_e128", N=2, L=130, S_real=190, E=128, causal=False, sink=True),
    W("dot_registers_window", L=300, S_real=300, n_reg=5, window=50),
    # windows wider than a workgroup's rows plus a tile: whole-tile steps run
    # between the masked steps on both sides
    W("dot_wide_window_registers", L=700, S_real=700, window=300, n_reg=3),
    # E = 128 dot mode runs 32-key tiles: register rows over two tiles, a window
    # edge inside a tile, a sink; and a non-causal ragged case with a few registers
    W("dot_registers_window_sink_e128", Hq=4, Hkv=2, L=270, S_real=270, E=128, n_reg=40, window=100, sink=True),
    W("dot_noncausal_registers_e128", N=2, L=90, S_real=150, E=128, n_reg=3, causal=False),
    W("dot_negative_scale_registers_e128", L=100, S_real=130, E=128, n_reg=33, scale=-0.07),
    # the lazy reference max: a large positive scale moves it on most tiles (the
    # half-row max passing the raw-score threshold), a tiny one never after the
    # first tile (threshold (m + 8) / c of order 1e5 against raw scores of order 10)
    W("dot_large_scale_rescales_e128", Hq=4, Hkv=2, L=333, S_real=333, E=128, scale=0.9, sink=True),
    W("dot_tiny_scale_e128", L=200, S_real=260, E=128, scale=1e-4),
    W("dot_large_scale_rescales_e64", N=2, L=300, S_real=300, scale=1.5, n_reg=5),
    W("rbf_wide_window_sink_e128", L=650, S_real=650, E=128, mode="rbf", window=260, sink=True, gamma=0.05),
    W("dot_single_query", N=3, Hq=4, Hkv=1, L=1, S_real=999, E=128),
    W("rbf_causal_registers", L=300, S_real=300, mode="rbf", n_reg=4, k_dist="dir_lognormal"),
    W("rbf_noncausal_many_registers_e128", L=130, S_real=90, E=128, mode="rbf", n_reg=70, causal=False),
    W("rbf_window_gqa_sink", Hq=4, Hkv=2, L=333, S_real=333, mode="rbf", window=100, sink=True, gamma=0.05),
    W("rbf_L_lt_S_e128", L=77, S_real=400, E=128, mode="rbf", gamma=0.02),
    W("f32_rbf_causal", dtype="f32", Hq=1, Hkv=1, L=256, S_real=256, mode="rbf"),
    W("f32_dot_window_gqa_sink_e128", dtype="f32", Hq=4, Hkv=2, L=100, S_real=100, E=128, window=30, sink=True),
    W("f32_rbf_registers_L_lt_S", dtype="f32", L=70, S_real=150, mode="rbf", n_reg=3, gamma=0.05),
    W("f32_dot_L_gt_S", dtype="f32", L=90, S_real=40, E=64),
    # fp32 RBF at E = 128: a key row's norm is summed over 32 staging lanes
    W("f32_rbf_e128_registers_window_sink", dtype="f32", Hq=2, Hkv=1, L=150, S_real=170, E=128, mode="rbf",
      n_reg=5, window=60, sink=True, gamma=0.05, k_dist="dir_lognormal"),
    W("f32_rbf_e128_noncausal_ragged", dtype="f32", N=2, L=70, S_real=333, E=128, mode="rbf", causal=False,
      gamma=0.02),
    # narrow causal windows at E = 64 (dot) with GQA groups of 4 or 8 heads take the
    # key-band kernel: L above and below S, ragged row counts and workgroups with
    # fewer than four query blocks, a one-key window with a negative scale, kv heads
    # spread over the XCDs (N * Hkv = 8) or not; groups of 1 and 2 heads stay on the
    # tiled kernel
    W("band_gqa4_L_lt_S_window128_sink", Hq=8, Hkv=2, L=300, S_real=777, window=128, sink=True),
    W("band_gqa8_L_gt_S_window100", N=2, Hq=16, Hkv=2, L=270, S_real=200, window=100),
    W("band_gqa4_window1_negative_scale", Hq=4, Hkv=1, L=150, S_real=150, window=1, scale=-0.1),
    W("band_gqa4_xcd_window127_sink", N=2, Hq=16, Hkv=4, L=333, S_real=333, window=127, sink=True),
    W("band_gqa8_window32_one_block", Hq=8, Hkv=1, L=31, S_real=64, window=32),
    W("band_gqa8_xcd_window128_sink", Hq=64, Hkv=8, L=700, S_real=700, window=128, sink=True),
    # logits with a spread of tens of units: the two-heads-per-wave path's
    # chunk maxima move its reference (the online rescale), positive and
    # negative scale (raw scores vs logits formed first)
    W("band_gqa8_large_logits_rescale", Hq=16, Hkv=2, L=300, S_real=300, window=128, scale=1.0, sink=True),
    W("band_gqa8_negative_large_logits", Hq=8, Hkv=1, L=200, S_real=260, window=100, scale=-1.0),
    W("tiled_gqa2_window64", Hq=4, Hkv=2, L=300, S_real=300, window=64, sink=True),
    # fp32 problems of 64 row tiles and more go to the tiled kernel (smaller ones to the
    # one-wave-per-row kernel, which every fp32 case above takes)
    W("f32_tiled_dot_causal_gqa_sink_e128", dtype="f32", N=2, Hq=8, Hkv=2, L=300, S_real=300, E=128, sink=True),
    W("f32_tiled_rbf_registers_window_e64", dtype="f32", Hq=16, Hkv=4, L=260, S_real=270, mode="rbf", n_reg=3,
      window=90, gamma=0.05, k_dist="dir_lognormal"),
    # one-wave-per-row kernel: rows longer than its 256-key chunk, a sink and registers
    W("f32_rows_long_noncausal_registers_sink", dtype="f32", Hq=2, Hkv=1, L=40, S_real=1300, n_reg=2,
      causal=False, sink=True),
]

# Wider shapes (hundreds of workgroups, more heads than the small cases) with
# ragged tails; checked on sampled rows.
PREFILL_WIDE_CASES = [
    W("wide_dot_causal_gqa_e128_ragged", Hq=64, Hkv=16, L=1000, S_real=1000, E=128),
    W("wide_dot_noncausal_sink_L_lt_S", N=2, Hq=48, Hkv=48, L=700, S_real=900, causal=False, sink=True),
    W("wide_rbf_causal_registers", Hq=64, Hkv=8, L=777, S_real=777, mode="rbf", n_reg=4, k_dist="dir_lognormal"),
    W("wide_rbf_noncausal_many_registers_sink_e128", Hq=128, Hkv=64, L=300, S_real=200, E=128, mode="rbf",
      n_reg=70, causal=False, sink=True, gamma=0.05),
    W("wide_dot_causal_L_gt_S_empty_rows_e128", Hq=96, Hkv=96, L=600, S_real=200, E=128),
    W("wide_dot_negative_scale_e128", Hq=128, Hkv=32, L=512, S_real=512, E=128, causal=False, scale=-0.06),
    W("wide_dot_causal_registers_e64", N=4, Hq=32, Hkv=4, L=520, S_real=520, n_reg=3, sink=True),
]

DECODE_CASES = [
    (W("dec_dot_sink_gqa4_e128", N=2, Hq=8, Hkv=2, L=1, S_real=5000, E=128, sink=True, decode=True), [0, 1, 3, 64]),
    (W("dec_rbf_registers", N=2, Hq=4, Hkv=2, L=1, S_real=3000, mode="rbf", n_reg=4, decode=True,
       k_dist="dir_lognormal"), [0, 7]),
    (W("dec_window_registers_sink", Hq=4, Hkv=1, L=1, S_real=4000, E=128, window=700, n_reg=4, sink=True,
       decode=True), [0, 2]),
    (W("dec_gqa20_two_query_groups", Hq=40, Hkv=2, L=1, S_real=1500, decode=True), [0]),
    (W("dec_mha_ragged", N=3, Hq=3, Hkv=3, L=1, S_real=777, decode=True, sink=True), [0, 5]),
    (W("dec_tiny_cache", Hq=4, Hkv=2, L=1, S_real=5, E=128, decode=True), [0, 3]),
]


@pytest.mark.parametrize("w", PREFILL_CASES, ids=[w.name for w in PREFILL_CASES])
def test_prefill_small(w):
    say(f"[prefill] {w}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    o, lse = run_gpu(w, q, k, v, sink)
    torch.cuda.synchronize()
    check(w, inp, o, lse)


@pytest.mark.parametrize("w", PREFILL_WIDE_CASES, ids=[w.name for w in PREFILL_WIDE_CASES])
def test_prefill_wide(w):
    say(f"[prefill wide] {w}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    o, lse = run_gpu(w, q, k, v, sink)
    torch.cuda.synchronize()
    check(w, inp, o, lse, rows=sample_rows(w, per_head=3, extra=128))


@pytest.mark.parametrize("w,splits", DECODE_CASES, ids=[c[0].name for c in DECODE_CASES])
def test_decode_small(w, splits):
    say(f"[decode] {w} splits={splits}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    for s in splits:
        o, lse = run_gpu(w, q, k, v, sink, num_splits=s)
        torch.cuda.synchronize()
        say(f"  num_splits={s}")
        check(w, inp, o, lse)


@pytest.mark.parametrize("E", [64, 128])
def test_prefill_constructed_logit_jumps(E):
    """Logits laid out per key so that every way out of the dot-mode weight check is
    taken: a run of keys about 6 log2 units above the first keys (weight sums of a tile
    past 2^8 while no row max passes the reference by more than 8: no rescale), one
    key 150 units up (weights against the old reference overflow: scores formed again,
    reference moved), then a ramp rising from there by 0.2 units per key (6.4 per
    32-key tile: weight sums fail the check on most tiles, the reference moves on some).
    q_i = u + noise, k_j = a_j u + noise, a_j set from the target logit."""
    w = W(f"dot_logit_jumps_e{E}", Hq=2, Hkv=1, L=600, S_real=600, E=E, scale=0.9 / np.sqrt(E))
    inp = gen.generate(w)
    r = np.random.default_rng(5)
    u = np.where(r.random(E) < 0.5, -1.0, 1.0).astype(np.float32)
    c = w.scale * np.log2(np.e) * float(u @ u)  # log2-unit logit per unit of a_j for q = u
    t = np.zeros(w.S_real)
    t[96:200] = 6.0
    t[333] = 150.0
    t[334:] = 150.0 + 0.2 * np.arange(1, w.S_real - 333)
    a = (t / c).astype(np.float32)
    q = u[None, None, None, :] + 0.05 * r.standard_normal((1, w.Hq, w.L, E)).astype(np.float32)
    k = a[None, None, :, None] * u + 0.05 * r.standard_normal((1, 1, w.S_real, E)).astype(np.float32)
    inp.q = gen.bf16_bits_from_f32(q)
    inp.k = gen.bf16_bits_from_f32(k)
    qd, kd, vd, sink = to_device(inp)
    o, lse = run_gpu(w, qd, kd, vd, sink)
    torch.cuda.synchronize()
    check(w, inp, o, lse)


def test_decode_matches_prefill_single_query():
    w = W("dec_vs_prefill", N=2, Hq=8, Hkv=2, L=1, S_real=2000, E=128, sink=True, decode=True)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    od, ld = run_gpu(w, q, k, v, sink, num_splits=9)
    of, lf = run_gpu(w.with_(decode=False), q, k, v, sink)
    torch.cuda.synchronize()
    assert (od.float() - of.float()).abs().max().item() <= 2e-2
    assert (ld - lf).abs().max().item() <= 1e-3


def test_empty_and_keyless_inputs():
    dev = "cuda:0"
    q = torch.zeros((0, 2, 5, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((0, 2, 7, 64), dtype=torch.bfloat16, device=dev)
    o, lse = attn.fwd(q, k, k)
    assert o.shape == q.shape and lse.shape == (0, 2, 5)
    # no keys at all: O = 0, LSE = -inf; with a sink, LSE = s_h
    q = torch.randn((1, 2, 5, 64), device=dev).to(torch.bfloat16)
    k = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    o, lse = attn.fwd(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    s = torch.tensor([0.25, -1.5], device=dev)
    o, lse = attn.fwd(q, k, k, causal=False, sink=s)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.allclose(lse, s[None, :, None].expand(1, 2, 5), atol=1e-6)


def test_outputs_stay_in_bounds_and_runs_are_deterministic():
    w = W("guard", Hq=4, Hkv=2, L=333, S_real=333, E=128, sink=True, window=100)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    n_o, n_l = q.numel(), w.N * w.Hq * w.L
    obuf = torch.full((n_o + 4096,), 7.0, dtype=torch.bfloat16, device="cuda:0")
    lbuf = torch.full((n_l + 1024,), 7.0, dtype=torch.float32, device="cuda:0")
    o1, l1 = attn.fwd(q, k, v, scale=w.scale, causal=True, window=w.window, sink=sink,
                      out=obuf[:n_o].view(q.shape), lse=lbuf[:n_l].view(w.N, w.Hq, w.L))
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = attn.fwd(q, k, v, scale=w.scale, causal=True, window=w.window, sink=sink)
    torch.cuda.synchronize()
    assert torch.all(obuf[n_o:] == 7.0) and torch.all(lbuf[n_l:] == 7.0)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    check(w, inp, o1, l1)


def test_binding_raises_on_misuse():
    q = torch.zeros((1, 6, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((1, 4, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(attn.AttnError) as ei:
        attn.fwd(q, k, k)
    assert ei.value.status == -2
    with pytest.raises(attn.AttnError) as ei:
        attn.fwd(q[:, :4], k, k, window=3, causal=False)
    assert ei.value.status == -4


# ----------------------------------------------------------------------------- full-size workloads


def _full(w, rows, splits=0):
    say(f"[full] {w.name}: generating inputs")
    inp = gen.generate(w)
    say(f"[full] {w.name}: running on the GPU")
    q, k, v, sink = to_device(inp)
    o, lse = run_gpu(w, q, k, v, sink, num_splits=splits)
    torch.cuda.synchronize()
    say(f"[full] {w.name}: oracle on {('all' if rows is None else len(rows))} rows")
    check(w, inp, o, lse, rows=rows)


def test_full_c1_rbf_causal_f32():
    _full(configs.C1, None)


def test_full_c2_dot_causal_bf16():
    _full(configs.C2, sample_rows(configs.C2))


def test_full_c3_rbf_causal_registers_bf16():
    _full(configs.C3, sample_rows(configs.C3, per_head=6))


def test_full_c4_sink_window_gqa_bf16():
    _full(configs.C4, sample_rows(configs.C4))


def test_full_c5_decode_splitk_bf16():
    _full(configs.C5, None)
