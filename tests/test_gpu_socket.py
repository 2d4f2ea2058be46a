"""GPU parity of SOCKET soft-LSH sparse decode (attn_socket_hash and
attn_socket_decode through the C ABI) against the fp64 oracle.

Bucket codes are integers decided by float32 projections computed the same way
on both sides (fused multiply-adds in element order), so they must match bit
for bit; value norms within 1e-5 relative.  The top-k set is unique only where
the k-th and (k+1)-th scores are apart: with the oracle's fp64 scores, every
key scoring above s_k (1 + 1e-4) must be chosen and every chosen key must score
at least s_k (1 - 1e-4) (s_k the k-th largest score); where no other key lies
in that band the chosen set must equal the oracle's and the output must match
the oracle's sparse attention within 2e-2 (O; 1e-4 for float32 caches) and
1e-3 (LSE).  Where scores tie within the band several selections are correct;
for every head the output must be exact attention (the oracle) over the keys
the GPU chose, to the same bars.
With top_k = S the sparse decode must equal the dense decode.

Exact ties: keys that are copies of one key (same K and V rows) get bit-equal
scores on both sides, so a selection whose only near-threshold keys are such a
group is fixed by the tie rule (lower index first) and compared exactly; the
cases reach every selection path (one read of the scores with and without the
scorer's histogram, ties straddling the cut, top_k above 4096, and more than
8192 keys in the threshold's first-level bin).
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_attn_amd as attn
from gpu_util import check_socket_heads, say, to_device
from workloads import gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu


def W(name, N, Hq, Hkv, S, E, mode="dot", sink=False, seed=51, k_dist="normal", gamma=0.05, dtype="bf16"):
    return Workload(name, dtype, N, Hq, Hkv, 1, S, E, mode, float(1.0 / np.sqrt(E)), float(gamma), True, 0, 0,
                    sink, True, seed, k_dist)


CASES = [
    (W("dot_gqa4_sink_e128", 2, 8, 2, 3000, 128, sink=True), 8, 6, 4.0, 200, (0, 3)),
    (W("rbf_e64_lognormal_keys", 1, 4, 4, 2500, 64, mode="rbf", k_dist="dir_lognormal"), 16, 4, 2.0, 333, (0,)),
    (W("gqa16_many_tables", 1, 16, 1, 1500, 64), 64, 2, 8.0, 64, (0,)),
    (W("ragged_small_budget_e128", 3, 4, 2, 777, 128, sink=True), 12, 5, 1.0, 17, (0, 2)),
    # packed 4-bit codes through the fast scorer (32 tables = one 16-byte chunk per key)
    (W("packed_fast_gqa4_e128", 2, 8, 2, 2048, 128, sink=True), 32, 4, 4.0, 150, (0,)),
    # packed 3-bit codes, odd table count (the last byte holds one code)
    (W("packed_odd_tables_e64", 1, 2, 1, 1000, 64), 7, 3, 2.0, 50, (0,)),
    # byte codes through the fast scorer
    (W("bytes_fast_gqa2_e64", 1, 4, 2, 1200, 64), 16, 5, 4.0, 100, (0,)),
    # float32 caches: codes from the float32 keys, exact fp32 attention over the choice (O bar 1e-4)
    (W("f32_dot_gqa4_sink_e128", 2, 8, 2, 3000, 128, sink=True, dtype="f32"), 8, 6, 4.0, 200, (0, 3)),
    (W("f32_rbf_e64_lognormal_keys", 1, 4, 4, 2500, 64, mode="rbf", k_dist="dir_lognormal", dtype="f32"), 16, 4,
     2.0, 333, (0,)),
    (W("f32_packed_fast_gqa4_e128", 1, 8, 2, 2048, 128, dtype="f32"), 32, 4, 4.0, 150, (0,)),
    (W("f32_bytes_odd_tables_e64", 1, 2, 1, 1000, 64, dtype="f32"), 7, 6, 2.0, 50, (0, 2)),
]


def _run(w, tables, bits, tau, top_k, splits, inp=None):
    inp = gen.generate(w) if inp is None else inp
    q, k, v, sink = to_device(inp)
    proj_np = gen.socket_projections(w.seed, tables, bits, w.E)
    proj = torch.from_numpy(proj_np).to("cuda:0")
    bk, vn = attn.socket_hash(k, v, proj, tables=tables, bits=bits)
    b_ref, vn_ref = oracle.socket_hash(inp.k, inp.v, proj_np, tables, bits)
    torch.cuda.synchronize()
    assert bk.shape[-1] == (tables + 1) // 2 if bits <= 4 else tables
    if bits <= 4 and tables % 2:  # the unused high nibble of the last byte is zero
        assert not (bk[..., -1] >> 4).any()
    assert np.array_equal(attn.unpack_codes(bk, tables, bits).cpu().numpy(), b_ref), "bucket codes differ"
    assert np.max(np.abs(vn.cpu().numpy() - vn_ref) / np.maximum(vn_ref, 1e-30)) < 1e-5
    o_ref, l_ref, sel_ref, sc_ref = oracle.socket_decode(inp.q, inp.k, inp.v, proj_np, b_ref, vn_ref, tables=tables,
                                                         bits=bits, tau=tau, top_k=top_k, mode=w.mode,
                                                         scale=w.scale, gamma=w.gamma, sink=inp.sink)
    outs = []
    for s in splits:
        o, lse, sel = attn.socket_decode(q, k, v, proj, bk, vn, tables=tables, bits=bits, tau=tau, top_k=top_k,
                                         scale=w.scale, mode=w.mode, gamma=w.gamma, sink=sink, num_splits=s,
                                         want_selected=True)
        torch.cuda.synchronize()
        outs.append((s, o, lse, sel))
    return inp, (o_ref, l_ref, sel_ref, sc_ref), outs


@pytest.mark.parametrize("w,tables,bits,tau,top_k,splits", CASES, ids=[c[0].name for c in CASES])
def test_socket_decode(w, tables, bits, tau, top_k, splits):
    say(f"[socket] {w.name} tables={tables} bits={bits} tau={tau} top_k={top_k}")
    inp, (o_ref, l_ref, sel_ref, sc_ref), outs = _run(w, tables, bits, tau, top_k, splits)
    for s, o, lse, sel in outs:
        og = o.float().cpu().numpy().astype(np.float64)
        lg = lse.cpu().numpy().astype(np.float64)
        sg = sel.cpu().numpy()
        unique = check_socket_heads(w, inp, top_k, sc_ref, sel_ref, o_ref, l_ref, og, lg, sg)
        say(f"  splits={s}: {unique}/{w.N * w.Hq} heads with a unique top-k; every head's output checked "
            f"against exact attention over its chosen keys")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_socket_full_budget_equals_dense_decode(dtype):
    w = W("full_budget", 2, 4, 2, 700, 128, sink=True, dtype=dtype)
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp)
    proj = torch.from_numpy(gen.socket_projections(w.seed, 4, 8, w.E)).to("cuda:0")
    bk, vn = attn.socket_hash(k, v, proj, tables=4, bits=8)
    o1, l1, sel = attn.socket_decode(q, k, v, proj, bk, vn, tables=4, bits=8, tau=1.0, top_k=700, sink=sink,
                                     num_splits=3, want_selected=True)
    o2, l2 = attn.decode(q, k, v, sink=sink, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(sel.cpu(), torch.arange(700, dtype=torch.int32).expand(2, 4, 700))
    assert (o1.float() - o2.float()).abs().max().item() <= (2e-2 if dtype == "bf16" else 1e-4)
    assert (l1 - l2).abs().max().item() <= 1e-3


def _tie_case(S, E, rank, group, extra_keep, seed, Hq=1, tables=16, bits=4, tau=2.0, identical=False):
    """A single-head cache where `group` other keys are copies of the key at `rank` (by the
    oracle's score) -- or, with identical=True, every key is a copy of key 0 -- and top_k cuts
    the copies after `extra_keep` of them."""
    w = W(f"ties_S{S}", 1, Hq, 1, S, E, seed=seed)
    inp = gen.generate(w)
    proj = gen.socket_projections(w.seed, tables, bits, E)
    k, v = inp.k.copy(), inp.v.copy()
    if identical:
        k[:, :, :] = k[:, :, :1]
        v[:, :, :] = v[:, :, :1]
        members = np.arange(S)
    else:
        b0, vn0 = oracle.socket_hash(k, v, proj, tables, bits)
        sc0 = oracle.socket_scores(inp.q[0, 0, 0], proj, b0[0, 0], vn0[0, 0], tables, bits, tau)
        src = int(np.lexsort((np.arange(S), -sc0))[rank])
        rest = np.setdiff1d(np.arange(S), [src])
        dup = np.random.default_rng(seed).choice(rest, size=group, replace=False)
        k[:, :, dup] = k[:, :, src:src + 1]
        v[:, :, dup] = v[:, :, src:src + 1]
        members = np.sort(np.concatenate([dup, [src]]))
    inp = gen.Inputs(w, inp.q, k, v, inp.sink)
    b, vn = oracle.socket_hash(k, v, proj, tables, bits)
    sc = oracle.socket_scores(inp.q[0, 0, 0], proj, b[0, 0], vn[0, 0], tables, bits, tau)
    tie = sc[members[0]]
    assert np.all(sc[members] == tie)
    top_k = int(np.sum(sc > tie)) + extra_keep
    near = np.abs(sc - tie) <= 1e-4 * tie
    assert np.array_equal(np.flatnonzero(near), members), "another key scores within the band of the copies"
    return w, inp, tables, bits, tau, top_k


TIE_CASES = [
    # name, S, E, rank of the copied key, copies, copies kept, seed, extra
    ("one_read_ties_straddle", 3000, 64, 120, 499, 250, 61, {}),
    ("one_read_ties_straddle_gqa2", 3000, 128, 90, 300, 77, 62, {"Hq": 2}),
    ("radix_top_k_above_4096", 12000, 64, 4000, 1999, 1000, 63, {}),
    ("radix_after_bin_overflow", 16000, 64, 150, 9000, 1000, 64, {}),
    ("all_keys_identical", 9000, 64, 0, 0, 100, 65, {"identical": True}),
]


@pytest.mark.parametrize("name,S,E,rank,group,keep,seed,extra", TIE_CASES, ids=[c[0] for c in TIE_CASES])
def test_socket_exact_ties(name, S, E, rank, group, keep, seed, extra):
    w, inp, tables, bits, tau, top_k = _tie_case(S, E, rank, group, keep, seed, **extra)
    say(f"[socket ties] {name}: S={S} top_k={top_k} Hq={w.Hq}")
    inp, (o_ref, l_ref, sel_ref, sc_ref), outs = _run(w, tables, bits, tau, top_k, (0,), inp=inp)
    for s, o, lse, sel in outs:
        sg = sel.cpu().numpy()
        og = o.float().cpu().numpy().astype(np.float64)
        lg = lse.cpu().numpy().astype(np.float64)
        # the copies were placed by head 0's ranking: its tie-broken selection is fixed by the rule
        assert np.array_equal(sg[0, 0], sel_ref[0, 0]), "tie-broken selection differs"
        check_socket_heads(w, inp, top_k, sc_ref, sel_ref, o_ref, l_ref, og, lg, sg)
