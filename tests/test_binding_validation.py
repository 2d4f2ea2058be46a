"""The Python binding rejects caller-supplied tensors that the C ABI cannot check
(it receives raw pointers): outputs, LSE, workspaces, SOCKET tables and hyperplanes
of the wrong shape, element type, device or layout.  A wrong one would make a
kernel read or write out of bounds, or through a host pointer.

CPU only: the binding's device type is pointed at "cpu" for these tests, and the
stream lookup (evaluated before every compute call into the library) is replaced
by one that fails, so a rejection that did not happen is reported without any
kernel being launched.
"""
import pytest
import torch

import softmax_attention_attn_amd as attn


class ReachedLibrary(Exception):
    pass


@pytest.fixture(autouse=True)
def cpu_binding(monkeypatch):
    monkeypatch.setattr(attn, "_DEVICE_TYPE", "cpu")

    def no_stream(*a, **k):
        raise ReachedLibrary("validation let the call through to the library")
    monkeypatch.setattr(attn, "_stream", no_stream)


N, Hq, Hkv, L, S, E = 2, 4, 2, 8, 16, 64
BF = torch.bfloat16


def qkv(L_=L):
    return (torch.zeros((N, Hq, L_, E), dtype=BF), torch.zeros((N, Hkv, S, E), dtype=BF),
            torch.zeros((N, Hkv, S, E), dtype=BF))


def meta(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="meta")


BAD_OUT = {
    "out_shape": lambda: dict(out=torch.zeros((N, Hq, L, E + 1), dtype=BF)),
    "out_dtype": lambda: dict(out=torch.zeros((N, Hq, L, E), dtype=torch.float32)),
    "out_layout": lambda: dict(out=torch.zeros((N, Hq, E, L), dtype=BF).transpose(2, 3)),
    "out_device": lambda: dict(out=meta((N, Hq, L, E), BF)),
    "lse_shape": lambda: dict(lse=torch.zeros((N, Hq, L + 1), dtype=torch.float32)),
    "lse_dtype": lambda: dict(lse=torch.zeros((N, Hq, L), dtype=torch.float64)),
    "lse_device": lambda: dict(lse=meta((N, Hq, L), torch.float32)),
    "lse_layout": lambda: dict(lse=torch.zeros((N, L, Hq), dtype=torch.float32).transpose(1, 2)),
}


def test_the_guard_itself_reports_a_call_that_gets_through():
    q, k, v = qkv()
    with pytest.raises(ReachedLibrary):
        attn.fwd(q, k, v)


@pytest.mark.parametrize("case", sorted(BAD_OUT))
def test_fwd_rejects_bad_outputs(case):
    q, k, v = qkv()
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, **BAD_OUT[case]())


def test_fwd_rejects_bad_key_len():
    q, k, v = qkv()
    for kl in (torch.zeros(N, dtype=torch.int64), torch.zeros(N + 1, dtype=torch.int32),
               meta((N,), torch.int32)):
        with pytest.raises(ValueError):
            attn.fwd(q, k, v, key_len=kl)


def test_fwd_rejects_inputs_off_the_device():
    q, k, v = qkv()
    with pytest.raises(ValueError):
        attn.fwd(q, meta(k.shape, BF), v)
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, sink=meta((Hq,), torch.float32))


def test_decode_rejects_bad_outputs():
    q, k, v = qkv(1)
    for bad in (dict(out=torch.zeros((N, Hq, 1, E + 1), dtype=BF)),
                dict(out=torch.zeros((N, Hq, 1, E), dtype=torch.float32)),
                dict(out=meta((N, Hq, 1, E), BF)),
                dict(out=torch.zeros((N, Hq, E, 2), dtype=BF).transpose(2, 3)[:, :, :1]),
                dict(lse=torch.zeros((N, Hq, 2), dtype=torch.float32)),
                dict(lse=torch.zeros((N, Hq, 1), dtype=torch.float64)),
                dict(lse=meta((N, Hq, 1), torch.float32))):
        with pytest.raises(ValueError):
            attn.decode(q, k, v, **bad)


def test_decode_rejects_workspace_off_the_device():
    q, k, v = qkv(1)
    with pytest.raises(ValueError):
        attn.decode(q, k, v, workspace=meta((1 << 20,), torch.uint8))
    with pytest.raises(ValueError):
        attn.decode(q, k, v, workspace=torch.zeros((2, 1 << 20), dtype=torch.uint8)[:, ::2])


def test_stream_decode_rejects_bad_outputs():
    q = torch.zeros((N, Hq, 1, E), dtype=BF)
    kc = torch.zeros((N, Hkv, 4 + 12, E), dtype=BF)
    vc = torch.zeros_like(kc)
    kw = dict(n_sink=4, window=12, pos=30)
    for bad in (dict(out=torch.zeros((N, Hq, 1, E), dtype=torch.float32)),
                dict(out=meta((N, Hq, 1, E), BF)),
                dict(lse=torch.zeros((N, Hq), dtype=torch.float32)),
                dict(workspace=meta((4096,), torch.uint8))):
        with pytest.raises(ValueError):
            attn.stream_decode(q, kc, vc, **kw, **bad)


def test_bwd_rejects_bad_tensors():
    q, k, v = qkv()
    o = torch.zeros_like(q)
    do = torch.zeros_like(q)
    lse = torch.zeros((N, Hq, L), dtype=torch.float32)
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse.double(), do)
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, meta((N, Hq, L), torch.float32), do)
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o[:, :, :4].contiguous(), lse, do)
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse, do, workspace=meta((4096,), torch.uint8))


TABLES, BITS = 6, 4
C = (TABLES + 1) // 2


def socket_tensors():
    q = torch.zeros((N, Hq, 1, E), dtype=BF)
    _, k, v = qkv()
    return dict(q=q, k=k, v=v, proj=torch.zeros((TABLES * BITS, E), dtype=torch.float32),
                buckets=torch.zeros((N, Hkv, S, C), dtype=torch.uint8),
                vnorm=torch.zeros((N, Hkv, S), dtype=torch.float32))


def test_socket_hash_rejects_bad_tensors():
    t = socket_tensors()
    for proj in (t["proj"].double(), t["proj"][:, :E - 1].contiguous(), meta(t["proj"].shape, torch.float32),
                 torch.zeros((E, TABLES * BITS), dtype=torch.float32).t()):
        with pytest.raises(ValueError):
            attn.socket_hash(t["k"], t["v"], proj, tables=TABLES, bits=BITS)
    with pytest.raises(ValueError):
        attn.socket_hash(meta(t["k"].shape, BF), t["v"], t["proj"], tables=TABLES, bits=BITS)
    with pytest.raises(ValueError):
        attn.socket_hash(t["k"], t["v"].float(), t["proj"], tables=TABLES, bits=BITS)


SOCKET_BAD = {
    "proj_dtype": ("proj", lambda t: t["proj"].double()),
    "proj_shape": ("proj", lambda t: torch.zeros((TABLES * BITS + 1, E), dtype=torch.float32)),
    "proj_device": ("proj", lambda t: meta(t["proj"].shape, torch.float32)),
    "buckets_dtype": ("buckets", lambda t: t["buckets"].to(torch.int8)),
    "buckets_shape": ("buckets", lambda t: torch.zeros((N, Hkv, S, TABLES), dtype=torch.uint8)),
    "buckets_device": ("buckets", lambda t: meta(t["buckets"].shape, torch.uint8)),
    "vnorm_dtype": ("vnorm", lambda t: t["vnorm"].double()),
    "vnorm_shape": ("vnorm", lambda t: torch.zeros((N, Hkv, S - 1), dtype=torch.float32)),
    "vnorm_device": ("vnorm", lambda t: meta(t["vnorm"].shape, torch.float32)),
}


@pytest.mark.parametrize("case", sorted(SOCKET_BAD))
def test_socket_decode_rejects_bad_tables(case):
    t = socket_tensors()
    name, make = SOCKET_BAD[case]
    t[name] = make(t)
    with pytest.raises(ValueError):
        attn.socket_decode(t["q"], t["k"], t["v"], t["proj"], t["buckets"], t["vnorm"], tables=TABLES, bits=BITS,
                           tau=1.0, top_k=4)


def test_socket_decode_rejects_bad_outputs():
    t = socket_tensors()
    for bad in (dict(out=torch.zeros((N, Hq, 1, E), dtype=torch.float32)),
                dict(lse=torch.zeros((N, Hq, 2), dtype=torch.float32)),
                dict(workspace=meta((1 << 16,), torch.uint8))):
        with pytest.raises(ValueError):
            attn.socket_decode(t["q"], t["k"], t["v"], t["proj"], t["buckets"], t["vnorm"], tables=TABLES,
                               bits=BITS, tau=1.0, top_k=4, **bad)


def test_valid_calls_pass_validation():
    # the guard above must be what stops these, not an over-eager check
    q, k, v = qkv()
    o = torch.zeros_like(q)
    lse = torch.zeros((N, Hq, L), dtype=torch.float32)
    calls = [
        lambda: attn.fwd(q, k, v, out=o, lse=lse, key_len=torch.full((N,), S, dtype=torch.int32)),
        lambda: attn.decode(q[:, :, :1].contiguous(), k, v, out=torch.zeros((N, Hq, 1, E), dtype=BF),
                            lse=torch.zeros((N, Hq, 1), dtype=torch.float32)),
        lambda: attn.bwd(q, k, v, o, lse, torch.zeros_like(q)),
        lambda: attn.stream_decode(q[:, :, :1].contiguous(), torch.zeros((N, Hkv, 16, E), dtype=BF),
                                   torch.zeros((N, Hkv, 16, E), dtype=BF), n_sink=4, window=12, pos=30),
    ]
    t = socket_tensors()
    calls.append(lambda: attn.socket_hash(t["k"], t["v"], t["proj"], tables=TABLES, bits=BITS))
    calls.append(lambda: attn.socket_decode(t["q"], t["k"], t["v"], t["proj"], t["buckets"], t["vnorm"],
                                            tables=TABLES, bits=BITS, tau=1.0, top_k=4))
    for c in calls:
        with pytest.raises(ReachedLibrary):
            c()
