"""Maximum sizes on the GPU, checked through properties that hold at any size
(no oracle call): with every key row zero all logits are equal, so each row's
output is the plain mean of the value rows it sees and its LSE is the log of
their count (plus the sink term when there is one).  Value rows are
v_j = (floor(j / 2^17) - 34) / 16 in every element, exact in bf16 and
changing every 131072 rows, so the expected means are exact fp64 sums and
reading any block of rows from the wrong place moves them.  The key/value slices are several GiB
(split-K decode: 9 M keys, 4.6 GB per tensor slice; bf16 prefill: 8 M keys,
just under the 2 GiB slice limit of its 32-bit tile offsets), so any 32-bit
offset arithmetic would read the wrong rows and move the mean.  Bars as
everywhere: 2e-2 on O, 1e-3 on LSE."""
import numpy as np
import pytest
import torch

import softmax_attention_attn_amd as attn
from gpu_util import say

pytestmark = pytest.mark.gpu


def _values(S, E, dev="cuda:0"):
    j = torch.arange(S, device=dev, dtype=torch.int64)
    col = (((j >> 17) - 34).to(torch.float32) / 16.0).to(torch.bfloat16)
    return col[:, None].expand(S, E).contiguous()


def _prefix_mean(S, upto):
    """fp64 mean of v_0 .. v_{upto-1} for each entry of upto."""
    v = ((np.arange(S, dtype=np.int64) >> 17) - 34) / 16.0
    c = np.concatenate([[0.0], np.cumsum(v)])
    upto = np.asarray(upto, dtype=np.int64)
    return c[upto] / upto


def test_decode_nine_million_keys():
    N, Hq, Hkv, S, E = 1, 4, 1, 9_000_000, 128
    say(f"[maxsize] decode S={S}")
    k = torch.zeros((N, Hkv, S, E), dtype=torch.bfloat16, device="cuda:0")
    v = _values(S, E).view(N, Hkv, S, E)
    q = torch.randn((N, Hq, 1, E), device="cuda:0").to(torch.bfloat16)
    o, lse = attn.decode(q, k, v, scale=1.0 / np.sqrt(E), causal=True)
    torch.cuda.synchronize()
    mean = _prefix_mean(S, [S])[0]
    eo = (o.float() - mean).abs().max().item()
    el = (lse.double() - np.log(S)).abs().max().item()
    say(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= 1e-3
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_eight_million_keys(causal):
    N, Hq, Hkv, L, S, E = 1, 2, 1, 100, 8_000_000, 128
    say(f"[maxsize] bf16 prefill L={L} S={S} causal={causal}")
    k = torch.zeros((N, Hkv, S, E), dtype=torch.bfloat16, device="cuda:0")
    v = _values(S, E).view(N, Hkv, S, E)
    q = torch.randn((N, Hq, L, E), device="cuda:0").to(torch.bfloat16)
    sink = torch.tensor([0.5, -1.0], device="cuda:0")
    o, lse = attn.fwd(q, k, v, scale=1.0 / np.sqrt(E), causal=causal, sink=sink)
    torch.cuda.synchronize()
    # bottom-right causal: row i sees keys 0 .. S - L + i
    cnt = (S - L + 1 + np.arange(L)) if causal else np.full(L, S)
    mean = _prefix_mean(S, cnt)
    s_h = sink.double().cpu().numpy()
    # the sink adds exp(s_h) to the denominator and nothing to the numerator (logits are 0)
    o_ref = mean[None, :] * cnt[None, :] / (cnt[None, :] + np.exp(s_h)[:, None])
    l_ref = np.log(cnt[None, :] + np.exp(s_h)[:, None])
    og = o.float().cpu().numpy().astype(np.float64)[0]
    eo = np.max(np.abs(og - o_ref[:, :, None]))
    el = np.max(np.abs(lse.cpu().numpy().astype(np.float64)[0] - l_ref))
    say(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= 1e-3
    del k, v
    torch.cuda.empty_cache()
