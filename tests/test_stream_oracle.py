"""Pins of the rolling-cache (StreamingLLM) part of the oracle, CPU only.

The kept set ("Attention Sink LLM..." page, section 3.2) is checked in closed
form; the gathered-rows decode is checked against the predicate form of the
oracle (registers = the sink tokens, sliding window, bottom-right causal), a
different code path, and against textbook cases; the ring-slot rule of
include/attn.h is checked by simulating appends.
"""
import numpy as np
import pytest

import oracle


def test_kept_positions_closed_form():
    for n_sink, window in ((4, 1), (4, 10), (0, 7), (3, 1000)):
        for pos in (0, 1, 3, 4, 5, 13, 14, 15, 100, 1000, 1013):
            kept = oracle.stream_kept_positions(n_sink, window, pos)
            if pos + 1 <= n_sink + window:
                assert np.array_equal(kept, np.arange(pos + 1))
            else:
                assert len(kept) == n_sink + window
                assert np.array_equal(kept[:n_sink], np.arange(n_sink))
                assert np.array_equal(kept[n_sink:], np.arange(pos - window + 1, pos + 1))


def slot(p, n_sink, window):
    return p if p < n_sink else n_sink + (p - n_sink) % window


@pytest.mark.parametrize("n_sink,window,chunks", [
    (4, 5, [1] * 30),
    (4, 5, [3, 2, 9, 1, 17, 4]),
    (0, 6, [2, 11, 1, 1, 30]),
    (2, 1, [1, 5, 1, 3]),
])
def test_ring_slots_hold_exactly_the_kept_tokens(n_sink, window, chunks):
    ring = [None] * (n_sink + window)
    pos = -1
    for T in chunks:
        first = pos + 1
        pos += T
        for p in range(first, pos + 1):  # what was kept after this append is written
            if p < n_sink or p > pos - window:
                ring[slot(p, n_sink, window)] = p
        rows = min(pos + 1, n_sink + window)
        assert sorted(ring[:rows]) == list(oracle.stream_kept_positions(n_sink, window, pos))
        assert all(x is None for x in ring[rows:])


def _hist(rng, N, Hq, Hkv, P, E):
    q = rng.standard_normal((N, Hq, 1, E))
    k = rng.standard_normal((N, Hkv, P, E))
    v = rng.standard_normal((N, Hkv, P, E))
    return q, k, v


@pytest.mark.parametrize("mode,n_sink,window,pos,sink", [
    ("dot", 4, 20, 100, False),
    ("dot", 4, 20, 10, True),      # nothing evicted yet
    ("rbf", 4, 8, 60, True),
    ("dot", 0, 16, 70, False),     # pure sliding window
    ("rbf", 2, 1, 33, False),      # window of one: the newest token plus the sinks
])
def test_gathered_decode_equals_predicate_form(mode, n_sink, window, pos, sink):
    rng = np.random.default_rng(5)
    N, Hq, Hkv, E = 2, 4, 2, 16
    q, k, v = _hist(rng, N, Hq, Hkv, pos + 1, E)
    s = rng.standard_normal(Hq) if sink else None
    o1, l1 = oracle.stream_decode(q, k, v, n_sink=n_sink, window=window, pos=pos, mode=mode, gamma=0.1, sink=s)
    # the same decode as "registers = sinks, real keys windowed", full history
    eff_sink = min(n_sink, pos + 1)
    o2, l2 = oracle.attn(q, k[:, :, :pos + 1], v[:, :, :pos + 1], mode=mode, gamma=0.1, causal=True,
                         window=window, n_reg=eff_sink, sink=s)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_no_eviction_is_plain_causal_decode():
    rng = np.random.default_rng(6)
    q, k, v = _hist(rng, 1, 2, 1, 30, 8)
    o1, l1 = oracle.stream_decode(q, k, v, n_sink=4, window=40, pos=29)
    o2, l2 = oracle.attn(q, k, v, causal=True)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_textbook_softmax_over_sinks_and_window():
    # brute force with explicit numpy: softmax over the logits of the kept keys
    rng = np.random.default_rng(7)
    E, pos, n_sink, window = 8, 25, 3, 5
    q, k, v = _hist(rng, 1, 1, 1, pos + 1, E)
    kept = [0, 1, 2, 21, 22, 23, 24, 25]
    z = np.array([q[0, 0, 0] @ k[0, 0, j] for j in kept]) / np.sqrt(E)
    w = np.exp(z - z.max())
    o_ref = (w[:, None] * v[0, 0, kept]).sum(0) / w.sum()
    lse_ref = z.max() + np.log(w.sum())
    o, lse = oracle.stream_decode(q, k, v, n_sink=n_sink, window=window, pos=pos)
    assert np.max(np.abs(o[0, 0, 0] - o_ref)) < 1e-12 and abs(lse[0, 0, 0] - lse_ref) < 1e-12
