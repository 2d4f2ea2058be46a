"""GPU parity on seeded random configurations: shapes, flags and scales drawn
from a fixed generator (so the set is the same on every run), each compared
with the fp64 oracle at the usual bars (bf16 O 2e-2, fp32 O 1e-4, LSE 1e-3;
gradients 2e-2 of max|g_ref|).  The draws mix what the hand-picked cases
cover one at a time: L below, equal to and above S, GQA group sizes, windows
narrower and wider than a tile, register rows, sinks, negative and large dot
scales, RBF with magnitude-skewed keys, fp32, single-query decode with forced
split counts, and the backward pass on the bf16 prefill draws."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import check, run_gpu, say, to_device
from workloads import gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu

N_DRAWS = 96


def _draw(i):
    r = np.random.default_rng(1000 + i)
    dtype = "f32" if r.random() < 0.2 else "bf16"
    E = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 8]))
    N = int(r.integers(1, 3))
    single = r.random() < 0.25
    decode = single and dtype == "bf16"  # split-K decode is bf16; an fp32 single query goes through attn_fwd
    S_real = int(r.integers(1, 420))
    L = 1 if single else int(r.integers(1, 420))
    mode = "rbf" if r.random() < 0.35 else "dot"
    causal = bool(r.random() < 0.7)
    window = int(r.integers(1, S_real + 80)) if causal and r.random() < 0.4 else 0
    n_reg = int(r.choice([0, 0, 1, 4, int(r.integers(1, 80))]))
    sink = bool(r.random() < 0.4)
    scale = float(r.choice([1.0, 1.0, -1.0, 3.0])) / np.sqrt(E)
    gamma = float(r.choice([0.02, 0.05, 0.125]))
    k_dist = "dir_lognormal" if mode == "rbf" and r.random() < 0.5 else "normal"
    name = (f"r{i:02d}_{dtype}_{mode}_e{E}_N{N}_{G * Hkv}to{Hkv}_L{L}_S{S_real}+{n_reg}"
            f"_{'c' if causal else 'nc'}_w{window}{'_sink' if sink else ''}{'_dec' if decode else ''}")
    w = Workload(name, dtype, N, G * Hkv, Hkv, L, S_real, E, mode, scale, gamma, causal, window, n_reg, sink,
                 decode, 500 + i, k_dist)
    splits = int(r.choice([0, 1, 3, 16])) if decode else 0
    return w, splits


DRAWS = [_draw(i) for i in range(N_DRAWS)]


@pytest.mark.parametrize("w,splits", DRAWS, ids=[d[0].name for d in DRAWS])
def test_random_forward(w, splits):
    say(f"[random] {w.name} splits={splits}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    o, lse = run_gpu(w, q, k, v, sink, num_splits=splits)
    torch.cuda.synchronize()
    check(w, inp, o, lse)


BWD_DRAWS = [d[0] for d in DRAWS if d[0].dtype == "bf16" and not d[0].decode]


@pytest.mark.parametrize("w", BWD_DRAWS, ids=[w.name for w in BWD_DRAWS])
def test_random_backward(w):
    say(f"[random bwd] {w.name}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    g = gen.bias_f32(w.seed + 100, (w.N, w.Hq, w.L, w.E))
    do_bits = gen.bf16_bits_from_f32(g)
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    kw = dict(scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window, n_reg=w.n_reg, sink=sink)
    o, lse = attn.fwd(q, k, v, **kw)
    dq, dk, dv, dsink = attn.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(inp.q, inp.k, inp.v, do_bits, mode=w.mode, scale=w.scale, gamma=w.gamma, causal=w.causal,
                          window=w.window, n_reg=w.n_reg, sink=inp.sink)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = t.float().cpu().numpy().astype(np.float64).reshape(-1, w.E)
        r = ref[name].reshape(-1, w.E)
        assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
        scale = max(np.abs(r).max(), 1e-6)
        err = np.abs(got - r).max() / scale
        say(f"  {name}: max|err|/max|ref| = {err:.3e}")
        assert err <= 2e-2, f"{w.name} {name}: {err:.3e}"
    if inp.sink is not None:
        ps = np.exp(inp.sink[None, :, None] - ref["lse"])
        bound = 1e-2 * np.sum(ps * np.abs(ref["delta"]), axis=(0, 2)) + 1e-6
        d = dsink.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(d - ref["dsink"]) <= bound)


# The general bias on random draws: float32 addends with -inf entries or
# boolean masks (with a fully masked row), broadcast over batch and/or head,
# with or without per-sequence key lengths.
def _bias_draw(i):
    w, _ = _draw(200 + i)
    w = w.with_(decode=False, L=max(w.L, 2), name=w.name.replace("_dec", "") + "_bias")
    r = np.random.default_rng(3000 + i)
    kind = [None, "f32", "bool"][int(r.integers(0, 3))]
    bn, bh = bool(r.random() < 0.5), bool(r.random() < 0.5)
    use_kl = bool(r.random() < 0.5) or kind is None
    p = float(r.choice([0.0, 0.1, 0.5]))
    return w, kind, bn, bh, use_kl, p


BIAS_DRAWS = [_bias_draw(i) for i in range(32)]


@pytest.mark.parametrize("w,kind,bn,bh,use_kl,p", BIAS_DRAWS, ids=[d[0].name for d in BIAS_DRAWS])
def test_random_biased_forward(w, kind, bn, bh, use_kl, p):
    say(f"[random bias] {w.name} kind={kind} per_batch={bn} per_head={bh} key_len={use_kl} p={p}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    b = None
    if kind is not None:
        shape = (w.N if bn else 1, w.Hq if bh else 1, w.L, w.S)
        if kind == "f32":
            b = gen.bias_f32(w.seed, shape, scale=1.0, p_neg_inf=p)
        else:
            b = gen.mask_bool(w.seed, shape, max(p, 0.3))
            b[..., 1, :] = False
    kl = gen.key_lengths(w.seed, w.N, w.S_real) if use_kl else None
    bt = None if b is None else torch.from_numpy(b).to("cuda:0")
    klt = None if kl is None else torch.from_numpy(kl).to("cuda:0")
    o, lse = attn.fwd(q, k, v, scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window,
                      n_reg=w.n_reg, sink=sink, bias=bt, key_len=klt)
    torch.cuda.synchronize()
    check(w, inp, o, lse, bias=b, key_len=kl)
