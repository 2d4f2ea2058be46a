"""GPU parity on seeded random configurations: shapes, flags and scales drawn
from a fixed generator (so the set is the same on every run), each compared
with the fp64 oracle at the usual bars (bf16 O 2e-2, fp32 O 1e-4, LSE 1e-3;
gradients 2e-2 of max|g_ref|).  The draws mix what the hand-picked cases
cover one at a time: L below, equal to and above S, GQA group sizes, windows
narrower and wider than a tile, register rows, sinks, negative and large dot
scales, RBF with magnitude-skewed keys, fp32, single-query decode with forced
split counts (bf16 and fp32), the backward pass on the prefill draws of both
element types (fp32 gradients within 1e-4 of max|g_ref|), and a quarter of the
SOCKET and rolling-cache draws with float32 caches."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import check, check_socket_heads, run_gpu, say, to_device
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
    decode = single
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


BWD_DRAWS = [d[0] for d in DRAWS if not d[0].decode]
BWD_TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}  # gradients (of max|g_ref|), d sink (of its sum)


@pytest.mark.parametrize("w", BWD_DRAWS, ids=[w.name for w in BWD_DRAWS])
def test_random_backward(w):
    say(f"[random bwd] {w.name}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    g = gen.bias_f32(w.seed + 100, (w.N, w.Hq, w.L, w.E))
    if w.dtype == "bf16":
        do_bits = gen.bf16_bits_from_f32(g)
        do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    else:
        do_bits = g
        do = torch.from_numpy(g).to("cuda:0")
    tol_g, tol_s = BWD_TOL[w.dtype]
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
        assert err <= tol_g, f"{w.name} {name}: {err:.3e}"
    if inp.sink is not None:
        ps = np.exp(inp.sink[None, :, None] - ref["lse"])
        bound = tol_s * np.sum(ps * np.abs(ref["delta"]), axis=(0, 2)) + 1e-6
        d = dsink.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(d - ref["dsink"]) <= bound)


# The key-band kernel (bf16, dot, causal window <= 128, E = 64, GQA groups of 4
# or 8, no registers) on random draws: L below, equal to and above S (rows
# with nothing visible), ragged block counts, windows from one key to 128,
# sinks, and dot scales from -2 to 2 (large ones move the reference max
# between the key-block chunks of the eight-heads path).
def _band_draw(i):
    r = np.random.default_rng(5000 + i)
    G = int(r.choice([4, 8]))
    Hkv = int(r.integers(1, 4))
    N = int(r.integers(1, 3))
    S_real = int(r.integers(1, 600))
    L = int(r.choice([S_real, int(r.integers(1, 600))]))
    window = int(r.choice([1, 31, 32, 33, 64, 100, 127, 128, int(r.integers(1, 129))]))
    sink = bool(r.random() < 0.5)
    scale = float(r.choice([0.125, 0.125, 1.0, 2.0, -0.125, -1.0]))
    name = f"b{i:02d}_N{N}_{G * Hkv}to{Hkv}_L{L}_S{S_real}_w{window}_s{scale}{'_sink' if sink else ''}"
    return Workload(name, "bf16", N, G * Hkv, Hkv, L, S_real, 64, "dot", scale, 0.125, True, window, 0, sink,
                    False, 7000 + i, "normal")


BAND_DRAWS = [_band_draw(i) for i in range(32)]


@pytest.mark.parametrize("w", BAND_DRAWS, ids=[w.name for w in BAND_DRAWS])
def test_random_band_forward(w):
    say(f"[random band] {w.name}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    o, lse = run_gpu(w, q, k, v, sink)
    torch.cuda.synchronize()
    check(w, inp, o, lse)


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


# SOCKET sparse decode on random draws: table counts and code widths (packed
# and byte codes, fast and generic scorers), temperatures, budgets from one key
# to every key, GQA groups, RBF keys.  Checked as in test_gpu_socket: bucket
# codes bit-exact, the chosen set valid around the k-th score (fp64 scores),
# and equal to the oracle's, with the output at the forward bars, wherever the
# top-k set is unique.
def _socket_draw(i):
    r = np.random.default_rng(5000 + i)
    E = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 3))
    G = int(r.choice([1, 2, 4, 8, 16]))
    N = int(r.integers(1, 3))
    S = int(r.choice([int(r.integers(1, 64)), int(r.integers(64, 2000)), int(r.integers(2000, 12000))]))
    mode = "rbf" if r.random() < 0.3 else "dot"
    k_dist = "dir_lognormal" if mode == "rbf" and r.random() < 0.5 else "normal"
    sink = bool(r.random() < 0.5)
    tables = int(r.choice([1, 3, 8, 16, 32, 64]))
    bits = int(r.integers(1, 9))
    tau = float(r.choice([0.5, 1.0, 2.0, 4.0, 8.0]))
    top_k = int(r.choice([1, max(1, S // 50), max(1, S // 4), S, int(r.integers(1, S + 1))]))
    splits = int(r.choice([0, 0, 1, 3]))
    dtype = "f32" if i % 4 == 3 else "bf16"
    name = (f"s{i:02d}_{dtype}_{mode}_e{E}_N{N}_{G * Hkv}to{Hkv}_S{S}_t{tables}b{bits}_tau{tau}_k{top_k}"
            f"{'_sink' if sink else ''}")
    w = Workload(name, dtype, N, G * Hkv, Hkv, 1, S, E, mode, float(1.0 / np.sqrt(E)), 0.05, True, 0, 0, sink,
                 True, 900 + i, k_dist)
    return w, tables, bits, tau, top_k, splits


SOCKET_DRAWS = [_socket_draw(i) for i in range(32)]


@pytest.mark.parametrize("w,tables,bits,tau,top_k,splits", SOCKET_DRAWS, ids=[d[0].name for d in SOCKET_DRAWS])
def test_random_socket(w, tables, bits, tau, top_k, splits):
    say(f"[random socket] {w.name} splits={splits}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    proj_np = gen.socket_projections(w.seed, tables, bits, w.E)
    proj = torch.from_numpy(proj_np).to("cuda:0")
    bk, vn = attn.socket_hash(k, v, proj, tables=tables, bits=bits)
    b_ref, vn_ref = oracle.socket_hash(inp.k, inp.v, proj_np, tables, bits)
    torch.cuda.synchronize()
    assert np.array_equal(attn.unpack_codes(bk, tables, bits).cpu().numpy(), b_ref), "bucket codes differ"
    assert np.max(np.abs(vn.cpu().numpy() - vn_ref) / np.maximum(vn_ref, 1e-30)) < 1e-5
    kw = dict(tables=tables, bits=bits, tau=tau, top_k=top_k, scale=w.scale, mode=w.mode, gamma=w.gamma, sink=sink,
              num_splits=splits, want_selected=True)
    if (w.Hq // w.Hkv) * tables * (1 << bits) * 4 > 64 * 1024:
        # the documented limit of the scorer's LDS table: a loud error, nothing computed
        with pytest.raises(attn.AttnError, match="UNSUPPORTED"):
            attn.socket_decode(q, k, v, proj, bk, vn, **kw)
        say("  rejected as documented (probability table over 64 KB)")
        return
    o_ref, l_ref, sel_ref, sc_ref = oracle.socket_decode(inp.q, inp.k, inp.v, proj_np, b_ref, vn_ref, tables=tables,
                                                         bits=bits, tau=tau, top_k=top_k, mode=w.mode,
                                                         scale=w.scale, gamma=w.gamma, sink=inp.sink)
    o, lse, sel = attn.socket_decode(q, k, v, proj, bk, vn, **kw)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    sg = sel.cpu().numpy()
    unique = check_socket_heads(w, inp, top_k, sc_ref, sel_ref, o_ref, l_ref, og, lg, sg)
    say(f"  {unique}/{w.N * w.Hq} heads with a unique top-k; every head checked over its chosen keys")


# Rolling (StreamingLLM) cache on random draws: sink and window sizes, chunk
# sequences mixing single tokens with chunks that cross the sink boundary or
# exceed the window; after every append the kept rows must be bit copies of
# the history and the newest token's decode must match the oracle.
def _stream_draw(i):
    r = np.random.default_rng(7000 + i)
    E = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 3))
    G = int(r.choice([1, 2, 4, 8]))
    N = int(r.integers(1, 3))
    n_sink = int(r.choice([0, 1, 4, int(r.integers(0, 20))]))
    window = int(r.choice([1, int(r.integers(1, 64)), int(r.integers(64, 600))]))
    chunks = []
    while len(chunks) < 10:
        chunks.append(int(r.choice([1, 1, int(r.integers(1, 40)), int(r.integers(1, window + n_sink + 50))])))
    P = sum(chunks)
    mode = "rbf" if r.random() < 0.3 else "dot"
    sink = bool(r.random() < 0.5)
    splits = int(r.choice([0, 0, 1, 5]))
    dtype = "f32" if i % 4 == 1 else "bf16"
    name = f"st{i:02d}_{dtype}_{mode}_e{E}_N{N}_{G * Hkv}to{Hkv}_sink{n_sink}_win{window}_P{P}{'_lsink' if sink else ''}"
    w = Workload(name, dtype, N, G * Hkv, Hkv, P, P, E, mode, float(1.0 / np.sqrt(E)), 0.05, True, 0, 0, sink,
                 False, 1100 + i, "normal")
    return w, n_sink, window, chunks, splits


STREAM_DRAWS = [_stream_draw(i) for i in range(16)]


@pytest.mark.parametrize("w,n_sink,window,chunks,splits", STREAM_DRAWS, ids=[d[0].name for d in STREAM_DRAWS])
def test_random_stream(w, n_sink, window, chunks, splits):
    say(f"[random stream] {w.name} chunks={chunks} splits={splits}")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    C = n_sink + window
    kc = torch.zeros((w.N, w.Hkv, C, w.E), dtype=k.dtype, device="cuda:0")
    vc = torch.full((w.N, w.Hkv, C, w.E), 1000.0, dtype=k.dtype, device="cuda:0")
    bits = torch.int16 if k.dtype == torch.bfloat16 else torch.int32
    tol_o = 2e-2 if w.dtype == "bf16" else 1e-4
    pos = -1
    for T in chunks:
        first = pos + 1
        pos += T
        attn.stream_append(k[:, :, first:pos + 1].contiguous(), v[:, :, first:pos + 1].contiguous(), kc, vc,
                           n_sink=n_sink, window=window, pos=first)
        kept = oracle.stream_kept_positions(n_sink, window, pos)
        slots = [p if p < n_sink else n_sink + (p - n_sink) % window for p in (int(x) for x in kept)]
        torch.cuda.synchronize()
        assert torch.equal(kc[:, :, slots].view(bits), k[:, :, torch.as_tensor(kept)].view(bits))
        assert torch.equal(vc[:, :, slots].view(bits), v[:, :, torch.as_tensor(kept)].view(bits))
        o_ref, l_ref = oracle.stream_decode(inp.q[:, :, pos:pos + 1], inp.k, inp.v, n_sink=n_sink, window=window,
                                            pos=pos, mode=w.mode, scale=w.scale, gamma=w.gamma, sink=inp.sink)
        o, lse = attn.stream_decode(q[:, :, pos:pos + 1].contiguous(), kc, vc, n_sink=n_sink, window=window, pos=pos,
                                    scale=w.scale, mode=w.mode, gamma=w.gamma, sink=sink, num_splits=splits)
        torch.cuda.synchronize()
        assert np.max(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref)) <= tol_o
        assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - l_ref)) <= 1e-3
