"""GPU parity of the rolling (StreamingLLM) cache: attn_stream_append and
attn_stream_decode through the C ABI against the fp64 oracle.

A token history is generated once; it is appended to a rolling cache in chunks
of mixed sizes (single tokens, chunks that cross the sink boundary, chunks
longer than the window), and after every append the newest token's query is
decoded against the cache.  Checks: the cache rows of every kept position are
bit-identical to the history rows (the append is a copy), rows of evicted
tokens are never read (the cache starts filled with values that would move the
output far outside the tolerance), and the decode output matches the oracle's
decode over the kept positions of the full history within 2e-2 (O) and 1e-3
(LSE).
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import TOL_LSE, TOL_O, say, to_device
from workloads import gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu


def H(name, P, dtype="bf16", N=1, Hq=4, Hkv=2, E=64, mode="dot", sink=False, seed=21, k_dist="normal",
      gamma=0.125):
    # a history of P tokens: q (N,Hq,P,E), k and v (N,Hkv,P,E)
    return Workload(name, dtype, N, Hq, Hkv, P, P, E, mode, float(1.0 / np.sqrt(E)), float(gamma), True, 0, 0,
                    sink, False, seed, k_dist)


def slot(p, n_sink, window):
    return p if p < n_sink else n_sink + (p - n_sink) % window


CASES = [
    (H("dot_gqa4_sink_e128", 274, N=2, Hq=8, Hkv=2, E=128, sink=True), 4, 50,
     [3, 1, 1, 60, 1, 200, 7, 1], (0, 1, 5)),
    (H("rbf_registers_lognormal_keys", 410, Hq=4, Hkv=4, mode="rbf", k_dist="dir_lognormal"), 4, 64,
     [1, 1, 1, 1, 1, 100, 1, 1, 64, 65, 1, 173], (0, 3)),
    (H("dot_pure_window_gqa8", 77, Hq=16, Hkv=2), 0, 33, [40, 1, 1, 33, 2], (0,)),
    (H("dot_long_window_e128", 2203, N=2, Hq=4, Hkv=1, E=128, sink=True), 4, 2000, [1500, 1, 700, 1, 1], (0, 2)),
    (H("dot_window_one", 12, Hq=2, Hkv=1), 2, 1, [1, 1, 1, 5, 1, 3], (0,)),
]


@pytest.mark.parametrize("w,n_sink,window,chunks,splits", CASES, ids=[c[0].name for c in CASES])
def test_stream_append_and_decode(w, n_sink, window, chunks, splits):
    say(f"[stream] {w.name} n_sink={n_sink} window={window} chunks={chunks} splits={splits}")
    assert sum(chunks) == w.L
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    N, Hkv, E = w.N, w.Hkv, w.E
    C = n_sink + window
    # rows that are never written hold k = 0, v = 1000: reading one would be obvious
    kc = torch.zeros((N, Hkv, C, E), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.full((N, Hkv, C, E), 1000.0, dtype=torch.bfloat16, device="cuda:0")
    pos = -1
    for T in chunks:
        first = pos + 1
        pos += T
        attn.stream_append(k[:, :, first:pos + 1].contiguous(), v[:, :, first:pos + 1].contiguous(), kc, vc,
                           n_sink=n_sink, window=window, pos=first)
        kept = oracle.stream_kept_positions(n_sink, window, pos)
        slots = [slot(int(p), n_sink, window) for p in kept]
        torch.cuda.synchronize()
        assert torch.equal(kc[:, :, slots].view(torch.int16), k[:, :, torch.as_tensor(kept)].view(torch.int16))
        assert torch.equal(vc[:, :, slots].view(torch.int16), v[:, :, torch.as_tensor(kept)].view(torch.int16))
        qq = q[:, :, pos:pos + 1].contiguous()
        o_ref, l_ref = oracle.stream_decode(inp.q[:, :, pos:pos + 1], inp.k, inp.v, n_sink=n_sink, window=window,
                                            pos=pos, mode=w.mode, scale=w.scale, gamma=w.gamma, sink=inp.sink)
        for s in splits:
            o, lse = attn.stream_decode(qq, kc, vc, n_sink=n_sink, window=window, pos=pos, scale=w.scale,
                                        mode=w.mode, gamma=w.gamma, sink=sink, num_splits=s)
            torch.cuda.synchronize()
            eo = np.max(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref))
            el = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - l_ref))
            say(f"  pos={pos} splits={s}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
            assert eo <= TOL_O["bf16"] and el <= TOL_LSE


def test_stream_append_f32_is_a_copy():
    w = H("f32_history", 90, dtype="f32", N=2, Hkv=3, E=128)
    inp = gen.generate(w)
    _, k, v, _ = to_device(inp)
    n_sink, window = 3, 20
    kc = torch.full((2, 3, n_sink + window, 128), -7.0, device="cuda:0")
    vc = torch.full_like(kc, -7.0)
    pos = -1
    for T in (2, 5, 30, 1, 52):
        first = pos + 1
        pos += T
        attn.stream_append(k[:, :, first:pos + 1].contiguous(), v[:, :, first:pos + 1].contiguous(), kc, vc,
                           n_sink=n_sink, window=window, pos=first)
    torch.cuda.synchronize()
    kept = oracle.stream_kept_positions(n_sink, window, pos)
    slots = [slot(int(p), n_sink, window) for p in kept]
    assert torch.equal(kc[:, :, slots].view(torch.int32), k[:, :, torch.as_tensor(kept)].view(torch.int32))
    assert torch.equal(vc[:, :, slots].view(torch.int32), v[:, :, torch.as_tensor(kept)].view(torch.int32))


def test_stream_decode_matches_attn_decode_before_eviction():
    # while nothing has been evicted, the rolling cache is the plain cache
    w = H("no_eviction", 300, N=2, Hq=8, Hkv=4, E=128, sink=True)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    kc = torch.zeros((2, 4, 4 + 500, 128), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.zeros_like(kc)
    attn.stream_append(k, v, kc, vc, n_sink=4, window=500, pos=0)
    qq = q[:, :, 299:300].contiguous()
    o1, l1 = attn.stream_decode(qq, kc, vc, n_sink=4, window=500, pos=299, sink=sink, num_splits=3)
    o2, l2 = attn.decode(qq, k, v, sink=sink, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
