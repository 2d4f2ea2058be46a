"""Seeded input generator and workload accounting (CPU only)."""
import math

import numpy as np
import torch

from workloads import configs, gen


def small(w, **kw):
    d = dict(N=min(w.N, 2), L=min(w.L, 16), S_real=min(w.S_real, 24))
    d.update(kw)
    return w.with_(**d)


def test_reproducible_and_sliceable():
    w = small(configs.C4)
    a = gen.generate(w)
    b = gen.generate(w, threads=1)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.sink, b.sink)):
        assert np.array_equal(x, y)
    assert np.array_equal(gen.k_slice(w, 0, 3), a.k[0, 3])
    assert np.array_equal(gen.q_slice(w, 0, 17), a.q[0, 17])
    assert a.q.dtype == np.uint16 and a.sink.dtype == np.float32 and a.sink.shape == (64,)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0], np.float32)])
    mine = gen.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(gen.f32_from_bf16_bits(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_register_tokens():
    w = small(configs.C3)
    a = gen.generate(w)
    assert np.all(a.k[:, :, :w.n_reg] == 0)
    assert np.array_equal(a.v[0, :, :w.n_reg], a.v[1, :, :w.n_reg])  # shared across the batch
    vals = gen.f32_from_bf16_bits(a.v[0, :, :w.n_reg]).ravel()
    assert 0.005 < vals.std() < 0.05
    assert not np.all(a.k[:, :, w.n_reg:] == 0)


def test_dir_lognormal_key_norms():
    w = configs.C3.with_(N=1, Hq=2, Hkv=2, L=8, S_real=20000)
    k = gen.f32_from_bf16_bits(gen.k_slice(w, 0, 0)[w.n_reg:]).astype(np.float64)
    ln = np.log(np.sqrt((k * k).sum(-1)))
    assert abs(ln.mean()) < 0.05 and abs(ln.std() - 1.0) < 0.05


def test_logit_variance_is_head_dim():
    """Var(q.k) = d_k for iid unit-variance entries; scaling by 1/sqrt(d_k) brings it to 1
    ("어텐션 메커니즘" section 2.1; d_k = 64 gives a spread of about +-8)."""
    w = configs.C4.with_(L=4096, S_real=4096)
    q = gen.f32_from_bf16_bits(gen.q_slice(w, 0, 0)).astype(np.float64)
    k = gen.f32_from_bf16_bits(gen.k_slice(w, 0, 0)).astype(np.float64)
    d = np.sum(q * k, -1)
    assert abs(d.var() / 64.0 - 1.0) < 0.1
    assert abs((d * w.scale).var() - 1.0) < 0.1
    assert abs(d.std() - 8.0) < 0.5


def test_visible_pair_counts():
    want = {configs.C1: 32896, configs.C2: 2098176, configs.C3: 33591296,
            configs.C4: 1040448, configs.C5: 131072}
    for w, n in want.items():
        assert configs.visible_pairs_per_head(w) == n, w.name
    assert math.isclose(configs.algorithmic_flops(configs.C2), 6.875e10, rel_tol=1e-3)
    assert math.isclose(configs.algorithmic_bytes(configs.C5), 4.295e9, rel_tol=1e-3)
