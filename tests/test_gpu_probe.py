"""The HBM bandwidth probes (include/attn_probe.h) do the work they are timed
on: the copy reproduces its source bit for bit (including a ragged tail past
the 4-way unrolled part), and the read touches every 32-bit word exactly once,
so the XOR of the words it leaves in its sink equals the XOR of every word of
the source."""
import numpy as np
import pytest
import torch

import softmax_attention_attn_amd as attn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 24) + 16 * 1000, 3 * (1 << 26)])
def test_probe_copy_and_read(nbytes):
    g = torch.Generator().manual_seed(nbytes % 1000003)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    src = host.to("cuda:0")
    dst = torch.zeros_like(src)
    attn.probe_copy(src, dst)
    sink = attn.probe_read(src)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), host)
    folded = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert folded == np.bitwise_xor.reduce(host.numpy().view(np.uint32))
