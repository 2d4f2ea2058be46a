"""GPU parity of the float32 split-K decode (attn_decode, attn_stream_decode with
dt = f32) against the fp64 oracle.

The fp32 decode keeps every operand in fp32 (products on the vector ALUs for
one or two query heads per kv head, on fp32 MFMA for more), so it is held to
the fp32 bars: max-abs error 1e-4 on O and 1e-3 on the LSE.  Cases cover both
kernels and each query-slot width (GQA group sizes 1, 2, 3, 5, 16 and 20, the
last over two query groups), both head dimensions, both score
modes, sinks, windows and register rows, forced split counts (one split, odd
counts, more splits than keys so that some splits are empty), caches with no
key at all, and the rolling cache.
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import TOL_LSE, TOL_O, check, run_gpu, say, to_device
from workloads import gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu


def D(name, N=1, Hq=2, Hkv=2, S=64, E=64, mode="dot", scale=None, gamma=0.125, window=0, n_reg=0, sink=False,
      seed=41, k_dist="normal"):
    if scale is None:
        scale = 1.0 / np.sqrt(E)
    return Workload(name, "f32", N, Hq, Hkv, 1, S, E, mode, float(scale), float(gamma), True, window, n_reg, sink,
                    True, seed, k_dist)


CASES = [
    (D("f32_mha_e64", N=3, Hq=3, Hkv=3, S=777, sink=True), [0, 1, 5]),
    (D("f32_gqa2_e128", N=2, Hq=4, Hkv=2, S=2049, E=128), [0, 3]),
    (D("f32_gqa3_ragged_e64", Hq=6, Hkv=2, S=1001, window=300, n_reg=4), [0, 2]),
    (D("f32_gqa5_rbf_e128", Hq=10, Hkv=2, S=3000, E=128, mode="rbf", gamma=0.05, sink=True), [0, 7]),
    (D("f32_gqa16_sink_e128", N=2, Hq=32, Hkv=2, S=4000, E=128, sink=True), [0, 1, 64]),
    (D("f32_gqa20_two_query_groups", Hq=40, Hkv=2, S=1500), [0, 4]),
    (D("f32_rbf_registers_lognormal", N=2, Hq=4, Hkv=2, S=2500, mode="rbf", n_reg=5, k_dist="dir_lognormal"),
     [0, 9]),
    (D("f32_window_registers_sink_e128", Hq=4, Hkv=1, S=4000, E=128, window=700, n_reg=4, sink=True), [0, 2]),
    (D("f32_large_scale_e64", Hq=8, Hkv=4, S=1200, scale=1.5), [0, 3]),
    (D("f32_tiny_cache_more_splits_than_keys", Hq=4, Hkv=2, S=5, E=128), [0, 3, 16]),
    # the MFMA kernel with the RBF fold over log-normal keys and registers, and with a large scale
    (D("f32_gqa8_rbf_registers_lognormal_e64", Hq=16, Hkv=2, S=2500, mode="rbf", n_reg=5, k_dist="dir_lognormal"),
     [0, 5]),
    (D("f32_gqa4_large_scale_e128", N=2, Hq=8, Hkv=2, S=1700, E=128, scale=1.2, sink=True), [0, 3]),
]


@pytest.mark.parametrize("w,splits", CASES, ids=[c[0].name for c in CASES])
def test_decode_f32(w, splits):
    say(f"[decode f32] {w} splits={splits}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    assert q.dtype == torch.float32
    for s in splits:
        o, lse = run_gpu(w, q, k, v, sink, num_splits=s)
        torch.cuda.synchronize()
        say(f"  num_splits={s}")
        check(w, inp, o, lse)


def test_decode_f32_keyless():
    # no key at all: O = 0, LSE = -inf; with a sink, LSE = the sink logit
    q = torch.randn((2, 4, 1, 64), device="cuda:0")
    k = torch.zeros((2, 2, 0, 64), device="cuda:0")
    o, lse = attn.decode(q, k, k)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    s = torch.tensor([0.5, -1.0, 2.0, 0.0], device="cuda:0")
    o, lse = attn.decode(q, k, k, sink=s, num_splits=3)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.allclose(lse, s[None, :, None].expand(2, 4, 1), atol=1e-6)


def test_decode_f32_matches_prefill_f32_single_query():
    w = D("f32_dec_vs_prefill", N=2, Hq=8, Hkv=2, S=2000, E=128, sink=True, window=900, n_reg=2)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    od, ld = run_gpu(w, q, k, v, sink, num_splits=9)
    of, lf = run_gpu(w.with_(decode=False), q, k, v, sink)
    torch.cuda.synchronize()
    assert (od - of).abs().max().item() <= TOL_O["f32"]
    assert (ld - lf).abs().max().item() <= TOL_LSE
    check(w, inp, od, ld)


def _slot(p, n_sink, window):
    return p if p < n_sink else n_sink + (p - n_sink) % window


@pytest.mark.parametrize("mode,n_sink,window,chunks", [
    ("dot", 4, 50, [3, 1, 1, 60, 1, 200, 7, 1]),
    ("rbf", 0, 33, [40, 1, 1, 33, 2]),
])
def test_stream_decode_f32(mode, n_sink, window, chunks):
    P = sum(chunks)
    w = Workload(f"f32_stream_{mode}", "f32", 2, 8, 2, P, P, 128, mode, float(1.0 / np.sqrt(128)), 0.05, True, 0, 0,
                 True, False, 43)
    say(f"[stream f32] {w.name} n_sink={n_sink} window={window} chunks={chunks}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    C = n_sink + window
    # rows never written hold k = 0, v = 1000: reading one would be obvious
    kc = torch.zeros((w.N, w.Hkv, C, w.E), device="cuda:0")
    vc = torch.full((w.N, w.Hkv, C, w.E), 1000.0, device="cuda:0")
    pos = -1
    for T in chunks:
        first = pos + 1
        pos += T
        attn.stream_append(k[:, :, first:pos + 1].contiguous(), v[:, :, first:pos + 1].contiguous(), kc, vc,
                           n_sink=n_sink, window=window, pos=first)
        qq = q[:, :, pos:pos + 1].contiguous()
        o_ref, l_ref = oracle.stream_decode(inp.q[:, :, pos:pos + 1], inp.k, inp.v, n_sink=n_sink, window=window,
                                            pos=pos, mode=w.mode, scale=w.scale, gamma=w.gamma, sink=inp.sink)
        for s in (0, 3):
            o, lse = attn.stream_decode(qq, kc, vc, n_sink=n_sink, window=window, pos=pos, scale=w.scale,
                                        mode=w.mode, gamma=w.gamma, sink=sink, num_splits=s)
            torch.cuda.synchronize()
            eo = np.max(np.abs(o.cpu().numpy().astype(np.float64) - o_ref))
            el = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - l_ref))
            say(f"  pos={pos} splits={s}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
            assert eo <= TOL_O["f32"] and el <= TOL_LSE
