"""GPU parity of the general bias (attn_fwd_biased through the C ABI) against
the fp64 oracle: float32 biases with -inf entries, boolean masks (True =
attend) with fully masked rows, per-sequence key lengths, broadcasting over
batch and head, together with causal / window / registers / sink / GQA / RBF,
bf16 and float32, ragged tails.  Bar: 2e-2 (bf16) / 1e-4 (f32) on O, 1e-3 on
LSE, identical -inf pattern of LSE.
"""
import numpy as np
import pytest
import torch

import softmax_attention_attn_amd as attn
from gpu_util import check, sample_rows, say, to_device
from workloads import configs, gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu


def W(name, dtype="bf16", N=2, Hq=4, Hkv=2, L=130, S_real=130, E=64, mode="dot", scale=None, gamma=0.125,
      causal=True, window=0, n_reg=0, sink=False, seed=31, k_dist="normal"):
    if scale is None:
        scale = 1.0 / np.sqrt(E)
    return Workload(name, dtype, N, Hq, Hkv, L, S_real, E, mode, float(scale), float(gamma), causal, window,
                    n_reg, sink, False, seed, k_dist)


# (workload, bias kind ("f32" / "bool" / None), bias batch dim, bias head dim, key lengths?, p)
CASES = [
    (W("f32bias_causal_gqa_e128_ragged", Hq=6, Hkv=3, L=300, S_real=300, E=128), "f32", "N", "H", False, 0.05),
    (W("boolmask_noncausal_sink", L=150, S_real=190, causal=False, sink=True), "bool", "N", "1", False, 0.7),
    (W("f32bias_broadcast_rbf_registers_keylen", L=260, S_real=260, mode="rbf", n_reg=4,
       k_dist="dir_lognormal"), "f32", "1", "1", True, 0.0),
    (W("keylen_only_causal_e128", N=4, Hq=4, Hkv=4, L=200, S_real=200, E=128), None, None, None, True, 0.0),
    (W("keylen_only_rbf_sink", N=3, L=100, S_real=333, mode="rbf", sink=True, causal=False), None, None, None,
     True, 0.0),
    (W("boolmask_window_gqa_sink_keylen", Hq=8, Hkv=2, L=400, S_real=400, window=100, sink=True), "bool", "1",
     "H", True, 0.8),
    (W("f32bias_L_lt_S_negative_scale", L=77, S_real=400, E=128, scale=-0.05), "f32", "N", "1", False, 0.1),
    (W("boolmask_L_gt_S", L=200, S_real=70, E=128), "bool", "N", "H", False, 0.5),
    (W("f32_f32bias_keylen", dtype="f32", L=100, S_real=120, E=64, n_reg=3, sink=True), "f32", "N", "H", True, 0.1),
    (W("f32_boolmask_rbf_e128", dtype="f32", N=1, L=90, S_real=90, E=128, mode="rbf", window=30), "bool", "1",
     "1", False, 0.6),
    # 80 row tiles: the tiled fp32 kernel with a bias and key lengths
    (W("f32_tiled_f32bias_keylen_gqa", dtype="f32", N=2, Hq=8, Hkv=4, L=257, S_real=300, E=64, sink=True), "f32",
     "N", "H", True, 0.05),
]


def _bias(w, kind, bn, bh, p):
    if kind is None:
        return None
    shape = (w.N if bn == "N" else 1, w.Hq if bh == "H" else 1, w.L, w.S)
    if kind == "f32":
        return gen.bias_f32(w.seed, shape, scale=1.0, p_neg_inf=p)
    m = gen.mask_bool(w.seed, shape, p)
    m[..., 1, :] = False  # a fully masked row in every (batch, head) the mask covers
    return m


@pytest.mark.parametrize("w,kind,bn,bh,use_kl,p", CASES, ids=[c[0].name for c in CASES])
def test_biased_prefill(w, kind, bn, bh, use_kl, p):
    say(f"[bias] {w} kind={kind} dims=({bn},{bh}) key_len={use_kl}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    b = _bias(w, kind, bn, bh, p)
    kl = gen.key_lengths(w.seed, w.N, w.S_real) if use_kl else None
    bt = None if b is None else torch.from_numpy(b).to("cuda:0")
    klt = None if kl is None else torch.from_numpy(kl).to("cuda:0")
    o, lse = attn.fwd(q, k, v, scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window,
                      n_reg=w.n_reg, sink=sink, bias=bt, key_len=klt)
    torch.cuda.synchronize()
    check(w, inp, o, lse, bias=b, key_len=kl)


def test_biased_prefill_wide_sampled_rows():
    w = W("wide_f32bias_causal_keylen_e128", N=2, Hq=16, Hkv=4, L=1000, S_real=1000, E=128)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    b = gen.bias_f32(w.seed, (w.N, 1, w.L, w.S), scale=2.0, p_neg_inf=0.02)
    kl = np.array([1000, 613], dtype=np.int32)
    o, lse = attn.fwd(q, k, v, scale=w.scale, causal=True, bias=torch.from_numpy(b).to("cuda:0"),
                      key_len=torch.from_numpy(kl).to("cuda:0"))
    torch.cuda.synchronize()
    check(w, inp, o, lse, rows=sample_rows(w, per_head=6, extra=256), bias=b, key_len=kl)


def test_zero_bias_and_all_true_mask_match_plain_forward():
    w = W("identity_biases", Hq=8, Hkv=2, L=257, S_real=257, E=128, window=64, n_reg=2, sink=True)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    kw = dict(scale=w.scale, causal=True, window=w.window, n_reg=w.n_reg, sink=sink)
    o0, l0 = attn.fwd(q, k, v, **kw)
    # same kernel family (the general path) with neutral biases: results equal the plain path up to rounding
    o1, l1 = attn.fwd(q, k, v, bias=torch.zeros((w.L, w.S), device="cuda:0"), **kw)
    o2, l2 = attn.fwd(q, k, v, bias=torch.ones((w.L, w.S), dtype=torch.bool, device="cuda:0"), **kw)
    torch.cuda.synchronize()
    for o, l in ((o1, l1), (o2, l2)):
        assert (o.float() - o0.float()).abs().max().item() <= 2e-2
        assert (l - l0).abs().max().item() <= 1e-3


def test_full_b1_bias_and_key_padding_sampled_rows():
    w = configs.B1
    say(f"[full] {w.name}: generating inputs")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    o, lse = attn.fwd(q, k, v, scale=w.scale, causal=w.causal, bias=torch.from_numpy(inp.bias).to("cuda:0"),
                      key_len=torch.from_numpy(inp.key_len).to("cuda:0"))
    torch.cuda.synchronize()
    check(w, inp, o, lse, rows=sample_rows(w), bias=inp.bias, key_len=inp.key_len)
