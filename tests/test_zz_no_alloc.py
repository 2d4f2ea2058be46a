"""attn_decode_noalloc (the decode entry point that allocates nothing: its split
partials live in the library's static device scratch) against attn_decode with
a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, so the second
runs over what the first left in the shared scratch; each must equal attn_decode
on the same inputs bit for bit (same kernels, same split count), and so also be
within the decode bars of the fp64 oracle (2e-2 on bf16 O, 1e-4 on fp32 O, 1e-3
on LSE), which is checked too; the same pair of calls runs for fp32 inputs.  A third call at the long-context decode size (8 x 32 query heads
over 8 kv heads, 131072 keys) fills about half of the scratch.
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


def W(name, N, Hq, Hkv, S, E, mode="dot", sink=True, seed=31, window=0, n_reg=0, dtype="bf16"):
    return Workload(name, dtype, N, Hq, Hkv, 1, S, E, mode, float(1.0 / np.sqrt(E)), 0.05, True, window, n_reg,
                    sink, True, seed)


def _both(w, num_splits=0, oracle_check=True):
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    kw = dict(scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window, n_reg=w.n_reg, sink=sink,
              num_splits=num_splits)
    o1 = torch.empty_like(q)
    l1 = torch.empty((w.N, w.Hq, 1), dtype=torch.float32, device=q.device)
    attn.decode_noalloc(q, k, v, out=o1, lse=l1, **kw)
    o2, l2 = attn.decode(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs from attn_decode"
    assert torch.equal(l1, l2), "LSE differs from attn_decode"
    if oracle_check:
        o_ref, l_ref = oracle.attn_workload(inp)
        eo = float(np.max(np.abs(o1.float().cpu().numpy() - o_ref)))
        el = float(np.max(np.abs(l1.cpu().numpy() - l_ref)))
        say(f"  {w.name}: equal to attn_decode; against the oracle max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= (2e-2 if w.dtype == "bf16" else 1e-4) and el <= 1e-3
    return o1


def test_noalloc_two_calls_second_smaller():
    say("[noalloc] large then small")
    big = W("noalloc_big", 4, 32, 8, 50000, 128, seed=32)
    small = W("noalloc_small", 2, 6, 2, 3001, 64, mode="rbf", seed=33, window=700, n_reg=3)
    need_big = attn.decode_workspace_bytes(big.N, big.Hq, big.Hkv, big.S, big.E)
    assert need_big <= attn.DECODE_NOALLOC_SCRATCH_BYTES
    _both(big)
    _both(small)
    _both(small, num_splits=7)


def test_noalloc_f32_two_calls_second_smaller():
    say("[noalloc] f32: large then small")
    big = W("noalloc_f32_big", 2, 16, 4, 40000, 128, seed=34, dtype="f32")
    small = W("noalloc_f32_small", 1, 6, 2, 2001, 64, mode="rbf", seed=35, window=500, n_reg=3, dtype="f32")
    assert attn.decode_workspace_bytes(big.N, big.Hq, big.Hkv, big.S, big.E) <= attn.DECODE_NOALLOC_SCRATCH_BYTES
    _both(big)
    _both(small)
    _both(small, num_splits=5)


def test_noalloc_long_context_size():
    w = configs.C5
    say(f"[noalloc] {w.name}")
    assert attn.decode_workspace_bytes(w.N, w.Hq, w.Hkv, w.S, w.E) <= attn.DECODE_NOALLOC_SCRATCH_BYTES
    _both(w, oracle_check=False)


def test_noalloc_rejects_partials_beyond_the_scratch():
    w = W("noalloc_too_many_splits", 8, 32, 8, 4096, 128)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    o = torch.empty_like(q)
    lse = torch.empty((w.N, w.Hq, 1), dtype=torch.float32, device=q.device)
    splits = 4096  # 8*32*4096*(128+2)*4 bytes of partials > 8 MiB
    assert attn.decode_workspace_bytes(w.N, w.Hq, w.Hkv, w.S, w.E, num_splits=splits) > \
        attn.DECODE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(attn.AttnError, match="WORKSPACE"):
        attn.decode_noalloc(q, k, v, out=o, lse=lse, sink=sink, num_splits=splits)
