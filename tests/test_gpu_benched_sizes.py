"""GPU parity at the exact sizes the benchmark times for the SOCKET sparse decode
and the rolling (StreamingLLM) cache, in the launch configuration it uses.

SOCKET ("기술 요약: SOCKET" page, method steps 1-4, at its 100K+ token, ~33x
sparsity setting): the long-context decode cache (8 sequences, 32 query heads
over 8 kv heads, 131072 keys, E = 128, sink), 64 tables of 4-bit codes, tau 4,
top_k 3972.  The whole cache is hashed and decoded on the GPU; the oracle hashes
a few sampled (batch, kv head) slices (about a second each on the CPU), whose
codes must match bit for bit and whose query heads are checked head by head:
valid selection, equal to the oracle's where unique, and exact attention over
the chosen keys within 2e-2 (O) / 1e-3 (LSE).

Rolling cache ("Attention Sink LLM..." page, section 3.2): the same heads with
4 sink tokens and a 4092-token window, filled by appends of the sink tokens and
then of tokens near position 100000, so that appends cross the ring's wrap
point; after every append the kept rows must be bit copies of the history and
the newest token's decode must match the oracle's decode over the kept
positions.
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import check_socket_heads, say, to_device
from workloads import configs, gen

pytestmark = pytest.mark.gpu


def test_socket_at_benched_size():
    sw = configs.SOCKET1
    w = sw.base
    say(f"[benched socket] {sw.name}: generating the cache")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    proj_np = gen.socket_projections(w.seed, sw.tables, sw.bits, w.E)
    proj = torch.from_numpy(proj_np).to("cuda:0")
    bk, vn = attn.socket_hash(k, v, proj, tables=sw.tables, bits=sw.bits)
    o, lse, sel = attn.socket_decode(q, k, v, proj, bk, vn, tables=sw.tables, bits=sw.bits, tau=sw.tau,
                                     top_k=sw.top_k, scale=w.scale, mode=w.mode, gamma=w.gamma, sink=sink,
                                     want_selected=True)
    torch.cuda.synchronize()
    del k, v
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    sg = sel.cpu().numpy()
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    G = w.Hq // w.Hkv
    S = w.S
    sc_ref = np.zeros((w.N, w.Hq, S))
    sel_ref = np.zeros((w.N, w.Hq, sw.top_k), dtype=np.int64)
    o_ref = np.zeros((w.N, w.Hq, 1, w.E))
    l_ref = np.zeros((w.N, w.Hq, 1))
    heads = []
    for n, kh in ((0, 0), (3, 5), (7, 7)):
        b_ref, vn_ref = oracle.socket_hash(inp.k[n:n + 1, kh:kh + 1], inp.v[n:n + 1, kh:kh + 1], proj_np,
                                           sw.tables, sw.bits)
        codes = attn.unpack_codes(bk[n:n + 1, kh:kh + 1], sw.tables, sw.bits).cpu().numpy()
        assert np.array_equal(codes, b_ref), f"bucket codes differ in slice {(n, kh)}"
        vg = vn[n, kh].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(vg - vn_ref[0, 0]) / np.maximum(vn_ref[0, 0], 1e-30)) < 1e-5
        for h in range(kh * G, (kh + 1) * G):
            s = oracle.socket_scores(inp.q[n, h, 0], proj_np, b_ref[0, 0], vn_ref[0, 0], sw.tables, sw.bits, sw.tau)
            idx = oracle.socket_select(s, sw.top_k)
            sk = None if inp.sink is None else np.asarray(inp.sink, dtype=np.float64)[h:h + 1]
            oo, ll = oracle.attn(np.ascontiguousarray(inp.q[n:n + 1, h:h + 1]),
                                 np.ascontiguousarray(inp.k[n:n + 1, kh:kh + 1, idx]),
                                 np.ascontiguousarray(inp.v[n:n + 1, kh:kh + 1, idx]), mode=w.mode, scale=w.scale,
                                 gamma=w.gamma, sink=sk)
            sc_ref[n, h], sel_ref[n, h], o_ref[n, h], l_ref[n, h] = s, idx, oo[0, 0], ll[0, 0]
            heads.append((n, h))
        say(f"  slice (n={n}, kv head={kh}): codes and norms match")
    unique = check_socket_heads(w, inp, sw.top_k, sc_ref, sel_ref, o_ref, l_ref, og, lg, sg, heads=heads)
    say(f"  {unique}/{len(heads)} sampled heads with a unique top-k; every sampled head checked over its chosen keys")


def test_stream_at_benched_size():
    sw = configs.STREAM1
    N, Hq, Hkv, E = sw.N, sw.Hq, sw.Hkv, sw.E
    C = sw.n_sink + sw.window
    # Tokens that are ever appended: the sink tokens and a stretch ending at sw.pos.  The ring
    # slot of position p >= n_sink is n_sink + (p - n_sink) % window, which returns to slot
    # n_sink at p = 98212 (window 4092): the second chunk below crosses it.
    first_tail = sw.pos - 6000
    chunks = [(0, sw.n_sink), (first_tail, 5000), (first_tail + 5000, 700), (first_tail + 5700, 299),
              (sw.pos - 1, 1), (sw.pos, 1)]
    wrap = sw.n_sink + ((first_tail - sw.n_sink) // sw.window + 1) * sw.window
    assert first_tail < wrap < first_tail + 5000
    r = np.random.default_rng(606)
    positions = np.concatenate([np.arange(a, a + t) for a, t in chunks])
    # history rows only where tokens exist; other rows stay zero and are never read
    k_hist = np.zeros((N, Hkv, sw.pos + 1, E), dtype=np.uint16)
    v_hist = np.zeros_like(k_hist)
    k_hist[:, :, positions] = gen.bf16_bits_from_f32(r.standard_normal((N, Hkv, len(positions), E), dtype=np.float32))
    v_hist[:, :, positions] = gen.bf16_bits_from_f32(r.standard_normal((N, Hkv, len(positions), E), dtype=np.float32))
    sink_np = r.standard_normal(Hq).astype(np.float32)
    sink = torch.from_numpy(sink_np).to("cuda:0")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    # rows never written hold k = 0, v = 1000: reading one would be obvious
    kc = torch.zeros((N, Hkv, C, E), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.full((N, Hkv, C, E), 1000.0, dtype=torch.bfloat16, device="cuda:0")
    for a, t in chunks:
        say(f"[benched stream] append positions {a}..{a + t - 1}")
        attn.stream_append(dev(k_hist[:, :, a:a + t]), dev(v_hist[:, :, a:a + t]), kc, vc, n_sink=sw.n_sink,
                           window=sw.window, pos=a)
        p = a + t - 1
        if p < sw.n_sink:
            continue
        kept = oracle.stream_kept_positions(sw.n_sink, sw.window, p)
        assert np.all(np.isin(kept, positions))
        slots = [x if x < sw.n_sink else sw.n_sink + (x - sw.n_sink) % sw.window for x in (int(y) for y in kept)]
        q_np = gen.bf16_bits_from_f32(r.standard_normal((N, Hq, 1, E), dtype=np.float32))
        o, lse = attn.stream_decode(dev(q_np), kc, vc, n_sink=sw.n_sink, window=sw.window, pos=p, scale=sw.scale,
                                    mode=sw.mode, gamma=sw.gamma, sink=sink)
        torch.cuda.synchronize()
        kk = kc[:, :, slots].view(torch.int16).cpu().numpy().view(np.uint16)
        vv = vc[:, :, slots].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(kk, k_hist[:, :, kept]) and np.array_equal(vv, v_hist[:, :, kept]), \
            f"kept rows differ after the append ending at {p}"
        o_ref, l_ref = oracle.stream_decode(q_np, k_hist, v_hist, n_sink=sw.n_sink, window=sw.window, pos=p,
                                            mode=sw.mode, scale=sw.scale, gamma=sw.gamma, sink=sink_np)
        eo = float(np.max(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref)))
        el = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - l_ref)))
        say(f"  decode at {p} over {len(kept)} kept rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= 2e-2 and el <= 1e-3
