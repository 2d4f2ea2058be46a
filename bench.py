#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--extras all|none]

A step is one call of the library on one batch of synthetic inputs already
resident in HBM.  The headline workload is the causal bf16 prefill
N=4, H=16, L=S=2048, E=128 (dot_causal_bf16_4x16x2048x128); its value is
TFLOP/s over the visible (query, key) pairs, 4*E flops each.  The other
workloads are timed the same way and reported under "extras" (prefill in
TFLOP/s, decode in HBM GB/s over the K/V bytes read once), as is one step of
streaming decode over a rolling cache (append the newest token, decode it; HBM
GB/s over the kept rows read once) and the backward pass on the C2 and C3
shapes (TFLOP/s at 10*E flops per visible pair) and a SOCKET sparse decode step
on the long-context decode shape (HBM GB/s over the codes, norms and selected
rows; speedup over the dense decode).  Each timing is the mean over K
back-to-back calls between two events; a second pass with one event pair per
call gives the spread of single calls ("ms_spread": p10 / p50 / p90).

The CPU baseline leg times the fp64 oracle on a bounded sample of rows of the
headline workload (about 15 s) and of every other forward and decode workload
(about 4 s each), on this host's cores, and checks the GPU output on those rows
against it ("cpu_baseline" and "parity" of the line and of each extra).  Every
workload is warmed up for at least 200 ms before its K timed calls, so that no
timing falls in the clock ramp of the first calls.  The long-context decode
figure is repeated at top level under "decode" (the metric's second half).
"probe_peaks" holds what this GPU sustains on a bf16 GEMM, a device copy and a
read-only sum (vendor library work) and on the library's own streaming read and
copy probes, and each roofline entry gives its fraction of the probe peak of
its bound beside the fraction of the published one.

Prints ONE JSON line.  Only one GPU is used: --gpus above 1 exits with a
message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import configs, gen  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE_BF16 = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte where the two bounds meet
METRIC = "prefill TFLOP/s + decode HBM GB/s, as % of MI355X roofline, oracle-exact"

KERNEL_FILES = {
    "prefill_bf16": "softmax_attention_attn_amd/csrc/prefill_bf16.hip",
    "prefill_bf16_band": "softmax_attention_attn_amd/csrc/prefill_bf16_band.hip",
    "prefill_f32": "softmax_attention_attn_amd/csrc/prefill_f32.hip",
    "decode_bf16": "softmax_attention_attn_amd/csrc/decode_bf16.hip",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_of(w) -> str:
    """Source file (KERNEL_FILES key) of the kernel the library runs for this workload."""
    if w.decode:
        return "decode_bf16"
    if w.dtype != "bf16":
        return "prefill_f32"
    # the library's key-band kernel: narrow causal windows, E = 64, dot, GQA 4 or 8, nothing else
    band = (w.E == 64 and w.mode == "dot" and w.causal and 0 < w.window <= 128 and w.n_reg == 0
            and w.bias == "none" and not w.key_len and w.Hq // w.Hkv in (4, 8))
    return "prefill_bf16_band" if band else "prefill_bf16"


# Headers every kernel source includes: a change there changes the kernels too.
KERNEL_HEADERS = ("softmax_attention_attn_amd/csrc/device_common.h", "softmax_attention_attn_amd/csrc/tile_common.h",
                  "softmax_attention_attn_amd/csrc/kernels.h", "include/attn.h")


def source_sha(kernel: str) -> str:
    """sha256 (first 16 hex digits) of a kernel source followed by the shared headers."""
    h = hashlib.sha256()
    for path in (KERNEL_FILES[kernel],) + KERNEL_HEADERS:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on this source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != source_sha(kernel):
        return None
    return float(m_b.group(1))


def measured_mfma_busy(kernel: str, workload: str):
    """MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs' active cycles) from the
    committed counter summary, if it was taken on this source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__mfma_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"mfma_busy_fraction:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != source_sha(kernel):
        return None
    return float(m_b.group(1))


def default_rotation(w) -> int:
    """Buffer sets to cycle through so that HBM, not the 256 MB on-die cache, serves the inputs."""
    return 3 if (not w.decode and configs.algorithmic_bytes(w) < 256e6 and w.name == configs.C4.name) else 1


def to_device(inp, torch, dev):
    import numpy as np

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    sink = torch.from_numpy(inp.sink).to(dev) if inp.sink is not None else None
    return t(inp.q), t(inp.k), t(inp.v), sink


SPREAD = {}  # workload name -> per-call ms percentiles from the spread pass


def timed(name, call, steps: int, torch, dev):
    """Mean ms per call over `steps` back-to-back calls between two events on the
    launching stream; then a second pass with one event pair per call (at most 200
    calls) records the p10 / p50 / p90 of single calls in SPREAD[name]."""
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    n = min(steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        call(i)
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda f: per[min(n - 1, int(f * (n - 1) + 0.5))]
    SPREAD[name] = {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "calls": n}
    return ms


WARM_MS = 200.0  # every workload is warmed up for at least this long (clocks ramp up over the first calls)


def warm(call, warmup: int, torch):
    """At least `warmup` calls and at least WARM_MS of back-to-back calls."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t0) * 1e3 < WARM_MS:
        call(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def probe_peaks(torch, attn, n: int = 8192, nbytes: int = 1 << 30, device: str = "cuda:0"):
    """What this GPU sustains on plain work, beside the published peaks: a bf16
    GEMM 8192 x 8192 x 8192 (torch.matmul, i.e. the vendor BLAS) in TFLOP/s; a
    1 GiB device-to-device copy (torch) and a sum over 1 GiB of bf16 in GB/s;
    and the library's own streaming read and copy of 1 GiB (attn_probe_read,
    attn_probe_copy: the access pattern of the HBM-bound kernels).  Each is
    warmed up for WARM_MS, then timed over back-to-back calls."""
    dev = torch.device(device)
    stream = torch.cuda.current_stream(dev)
    out = {}

    def rate_of(call, calls):
        warm(lambda _i: call(), 3, torch)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(calls):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls

    x = torch.randn(n, n, device=dev).to(torch.bfloat16)
    y = torch.randn(n, n, device=dev).to(torch.bfloat16)
    z = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    ms = rate_of(lambda: torch.matmul(x, y, out=z), 20)
    out["bf16_gemm"] = {"value": 2.0 * n ** 3 / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                        "what": f"torch.matmul bf16 {n}x{n}x{n}", "ms": ms}
    del x, y, z
    nb = nbytes
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    ms = rate_of(lambda: dst.copy_(src), 20)
    out["hbm_copy"] = {"value": 2.0 * nb / (ms * 1e-3) / 1e9, "unit": "GB/s",
                       "what": f"{nb >> 20} MiB device copy, read + write bytes", "ms": ms}
    del dst
    xs = src.view(torch.bfloat16)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    ms = rate_of(lambda: torch.sum(xs, dim=0, dtype=torch.float32, out=acc), 20)
    out["hbm_read"] = {"value": nb / (ms * 1e-3) / 1e9, "unit": "GB/s",
                       "what": f"torch.sum over {nb >> 20} MiB of bf16, bytes read", "ms": ms}
    del xs, acc
    # The library's own probes: the 16-byte non-temporal access pattern of the
    # HBM-bound kernels (include/attn_probe.h).
    sink = attn.probe_read(src)
    ms = rate_of(lambda: attn.probe_read(src, sink=sink), 20)
    out["hbm_read_kernel"] = {"value": nb / (ms * 1e-3) / 1e9, "unit": "GB/s",
                              "what": f"attn_probe_read over {nb >> 20} MiB, bytes read", "ms": ms}
    dst = torch.empty_like(src)
    ms = rate_of(lambda: attn.probe_copy(src, dst), 20)
    out["hbm_copy_kernel"] = {"value": 2.0 * nb / (ms * 1e-3) / 1e9, "unit": "GB/s",
                              "what": f"attn_probe_copy of {nb >> 20} MiB, bytes read + written", "ms": ms}
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def attach_probe(entry: dict, probes) -> None:
    """Adds the probe peak of the entry's bound and the fraction of it reached (for
    HBM the best of the device copies and streaming reads)."""
    if not probes:
        return
    hbm = max((p for p in (probes.get(k) for k in ("hbm_copy", "hbm_read", "hbm_read_kernel", "hbm_copy_kernel"))
               if p), key=lambda p: p["value"], default=None)
    p = {"mfma": probes.get("bf16_gemm"), "hbm": hbm}.get(entry.get("bound"))
    if p is None or p["unit"] != entry.get("unit"):
        return
    entry["probe_peak"] = p["value"]
    entry["frac_of_probe"] = entry["achieved" if "achieved" in entry else "value"] / p["value"]


def time_workload(w, steps: int, warmup: int, rotate: int, torch, attn, keep_first_output=False):
    """Average ms per call over `steps` back-to-back calls, inputs resident in HBM."""
    dev = torch.device("cuda:0")
    log(f"[bench] {w.name}: generating inputs")
    t0 = time.time()
    inp = gen.generate(w)
    log(f"[bench] {w.name}: inputs ready in {time.time() - t0:.1f}s, copying to the GPU")
    q, k, v, sink = to_device(inp, torch, dev)
    ub = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
    kl = torch.from_numpy(inp.key_len).to(dev) if inp.key_len is not None else None
    sets = [(q, k, v)]
    for _ in range(max(0, rotate - 1)):
        sets.append((q.clone(), k.clone(), v.clone()))
    outs = [(torch.empty_like(q), torch.empty((w.N, w.Hq, w.L), dtype=torch.float32, device=dev))
            for _ in sets]
    kw = dict(scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window, n_reg=w.n_reg,
              sink=sink)
    ws = None
    if w.decode:
        nbytes = attn.decode_workspace_bytes(w.N, w.Hq, w.Hkv, w.S, w.E, w.causal, w.window, w.n_reg)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def call(i):
        qq, kk, vv = sets[i % len(sets)]
        oo, ll = outs[i % len(outs)]
        if w.decode:
            attn.decode(qq, kk, vv, workspace=ws, out=oo, lse=ll, **kw)
        else:
            attn.fwd(qq, kk, vv, out=oo, lse=ll, bias=ub, key_len=kl, **kw)

    call(0)
    torch.cuda.synchronize()
    first = (outs[0][0].clone(), outs[0][1].clone()) if keep_first_output else None
    warm(call, warmup, torch)
    ms = timed(w.name, call, steps, torch, dev)
    return ms, inp, first


def time_stream(sw, steps: int, warmup: int, rotate: int, torch, attn):
    """Average ms per streaming step (append the newest token, decode its query) over a
    rolling cache deep into the stream; `rotate` cache sets defeat the on-die cache."""
    dev = torch.device("cuda:0")
    log(f"[bench] {sw.name}: generating inputs")
    base = configs.Workload(sw.name, "bf16", sw.N, sw.Hq, sw.Hkv, 1, sw.rows, sw.E, sw.mode, sw.scale, sw.gamma,
                            True, 0, 0, sw.sink, True, sw.seed)
    q, kc, vc, sink = to_device(gen.generate(base), torch, dev)
    _, kn, vn, _ = to_device(gen.generate(base.with_(S_real=1, seed=sw.seed + 1000)), torch, dev)
    cap = sw.n_sink + sw.window
    if kc.shape[2] != cap:  # early in the stream: pad the cache to its capacity
        pad = torch.zeros((sw.N, sw.Hkv, cap - kc.shape[2], sw.E), dtype=kc.dtype, device=dev)
        kc, vc = torch.cat([kc, pad], 2).contiguous(), torch.cat([vc, pad], 2).contiguous()
    sets = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(max(0, rotate - 1))]
    o = torch.empty_like(q)
    lse = torch.empty((sw.N, sw.Hq, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, attn.stream_decode_workspace_bytes(sw.N, sw.Hq, sw.Hkv, sw.E, sw.n_sink, sw.window,
                                                                sw.pos)), dtype=torch.uint8, device=dev)
    kw = dict(n_sink=sw.n_sink, window=sw.window, pos=sw.pos)

    def call(i):
        k_c, v_c = sets[i % len(sets)]
        attn.stream_append(kn, vn, k_c, v_c, **kw)
        attn.stream_decode(q, k_c, v_c, scale=sw.scale, mode=sw.mode, gamma=sw.gamma, sink=sink, workspace=ws,
                           out=o, lse=lse, **kw)

    warm(call, warmup + 1, torch)
    return timed(sw.name, call, steps, torch, dev)


def time_backward(w, steps: int, warmup: int, torch, attn):
    """Average ms per backward step (all gradients of O for one upstream gradient); the
    forward that produces O and LSE runs once before timing."""
    dev = torch.device("cuda:0")
    log(f"[bench] {w.name} backward: generating inputs")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp, torch, dev)
    gbits = gen.bf16_bits_from_f32(gen.bias_f32(w.seed + 100, (w.N, w.Hq, w.L, w.E)))
    import numpy as np
    do = torch.from_numpy(gbits.view(np.int16)).view(torch.bfloat16).to(dev)
    kw = dict(scale=w.scale, mode=w.mode, gamma=w.gamma, causal=w.causal, window=w.window, n_reg=w.n_reg, sink=sink)
    o, lse = attn.fwd(q, k, v, **kw)
    ws = torch.empty(max(16, int(attn.load().attn_bwd_workspace_bytes(w.N, w.Hq, w.L))), dtype=torch.uint8,
                     device=dev)
    def call(_i):
        attn.bwd(q, k, v, o, lse, do, workspace=ws, **kw)

    warm(call, warmup + 1, torch)
    return timed(w.name + "__backward", call, steps, torch, dev)


def time_socket(sw, steps: int, warmup: int, torch, attn):
    """Average ms per SOCKET decode step (scores, top-k, sparse attention) on the base decode
    workload's cache, hashed once before timing."""
    dev = torch.device("cuda:0")
    w = sw.base
    log(f"[bench] {sw.name}: generating inputs")
    inp = gen.generate(w)
    q, k, v, sink = to_device(inp, torch, dev)
    proj = torch.from_numpy(gen.socket_projections(w.seed, sw.tables, sw.bits, w.E)).to(dev)
    buckets, vnorm = attn.socket_hash(k, v, proj, tables=sw.tables, bits=sw.bits)
    o = torch.empty_like(q)
    lse = torch.empty((w.N, w.Hq, 1), dtype=torch.float32, device=dev)
    need = int(attn.load().attn_socket_decode_workspace_bytes(w.N, w.Hq, w.Hkv, w.S, w.E, sw.tables, sw.bits,
                                                              sw.top_k, 0))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    kw = dict(tables=sw.tables, bits=sw.bits, tau=sw.tau, top_k=sw.top_k, scale=w.scale, sink=sink, workspace=ws,
              out=o, lse=lse)
    def call(_i):
        attn.socket_decode(q, k, v, proj, buckets, vnorm, **kw)

    warm(call, warmup + 1, torch)
    return timed(sw.name, call, steps, torch, dev)


def stream_rate(sw, ms: float):
    gbs = configs.stream_bytes(sw) / (ms * 1e-3) / 1e9
    return {"value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS}


def rate(w, ms: float):
    if w.decode:
        gbs = configs.algorithmic_bytes(w) / (ms * 1e-3) / 1e9
        return {"value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS}
    tf = configs.algorithmic_flops(w) / (ms * 1e-3) / 1e12
    gbs = configs.algorithmic_bytes(w) / (ms * 1e-3) / 1e9
    if w.dtype == "bf16" and configs.algorithmic_flops(w) / configs.algorithmic_bytes(w) < RIDGE_BF16:
        # Below the ridge point the kernel is bound by HBM, not by the matrix cores.
        return {"value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS,
                "tflops": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS}
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    out = {"value": tf, "unit": "TFLOP/s", "bound": "mfma" if w.dtype == "bf16" else "alu", "peak": peak,
           "frac": tf / peak}
    out["hbm_GBps"] = gbs
    out["hbm_frac"] = gbs / PEAK_HBM_GBS
    return out


def cpu_baseline(w, inp, o_gpu, lse_gpu, seconds: float):
    """Time the fp64 oracle on a bounded row sample (all rows when they fit the time budget);
    compare the GPU rows with it.  Returns (cpu_baseline, parity) dicts."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads(0)
    rng = np.random.default_rng(1234)
    total = w.N * w.Hq * w.L
    # probe the per-row cost, then size the sample to ~`seconds`
    probe = np.sort(rng.choice(total, size=min(total, 4 * threads), replace=False))
    t0 = time.perf_counter()
    oracle.attn_workload(inp, rows=probe, threads=threads)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = int(min(total, max(len(probe), len(probe) * seconds / dt)))
    rows = np.sort(rng.choice(total, size=n, replace=False))
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attn_workload(inp, rows=rows, threads=threads)
    el = time.perf_counter() - t0
    # algorithmic work of exactly these rows (visible pairs, padding keys excluded)
    off = w.S_real - w.L
    i = rows % w.L
    nn = rows // (w.Hq * w.L)
    kl = np.asarray(w.key_len, dtype=np.int64)[nn] if w.key_len else np.full_like(i, w.S_real)
    ip = i + off
    hi = np.minimum(kl - 1, ip) if w.causal else kl - 1
    lo = np.maximum(0, ip - w.window + 1) if w.window > 0 else np.zeros_like(i)
    pairs = float(np.maximum(0, hi - lo + 1).sum() + w.n_reg * len(rows))
    flops = 4.0 * w.E * pairs
    og = o_gpu.float().cpu().numpy().reshape(-1, w.E)[rows].astype(np.float64)
    lg = lse_gpu.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    eo = float(np.abs(og - o_ref).max())
    finite = np.isfinite(lse_ref)
    el_lse = float(np.abs(lg[finite] - lse_ref[finite]).max()) if finite.any() else 0.0
    same_inf = bool(np.array_equal(np.isneginf(lg), np.isneginf(lse_ref)))
    tol = 2e-2 if w.dtype == "bf16" else 1e-4
    if w.decode:
        # decode is priced in bytes: the K/V rows the sampled query heads read
        byts = float(len(rows) * (w.S * 2 * w.E * (2 if w.dtype == "bf16" else 4)))
        base = {"value": byts / el / 1e9, "unit": "GB/s"}
    else:
        base = {"value": flops / el / 1e12, "unit": "TFLOP/s"}
    base.update({"cores": threads, "kind": "oracle",
                 "sample": f"{len(rows)} of {total} output rows of {w.name} (seeded uniform sample), "
                           f"{pairs:.4g} visible pairs, {el:.2f}s wall, fp64, OpenMP over rows"})
    parity = {"rows": len(rows), "max_abs_err_o": eo, "max_abs_err_lse": el_lse, "tol_o": tol,
              "tol_lse": 1e-3, "pass": bool(eo <= tol and el_lse <= 1e-3 and same_inf)}
    return base, parity


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=configs.C2.name,
                    choices=sorted(configs.BY_NAME) + sorted(configs.STREAM_BY_NAME) + sorted(configs.SOCKET_BY_NAME) +
                    sorted(w.name + "__backward" for w in configs.BACKWARD))
    ap.add_argument("--extras", default="all", choices=["all", "none"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time budget for the headline workload's CPU baseline")
    ap.add_argument("--cpu-seconds-extra", type=float, default=4.0,
                    help="oracle time budget for each other forward / decode workload")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input/output buffer sets cycled through (0: 3 for workloads whose bytes fit the "
                         "256 MB on-die cache, else 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the probe-measured peaks (bf16 GEMM and device copy)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, time a plain device-to-device copy of this many bytes "
                         "(the reference kernel for calibrating HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the attention kernels run on one GPU's share and nothing here spans GPUs.", file=sys.stderr)
        return 2

    import torch

    import softmax_attention_attn_amd as attn
    attn.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            dst.copy_(src)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        print(json.dumps({"copy_bytes": args.copy_bytes, "ms": ms,
                          "GBps_read_plus_write": 2 * args.copy_bytes / (ms * 1e-3) / 1e9}), flush=True)
        return 0

    if args.workload.endswith("__backward"):
        bw = configs.BY_NAME[args.workload[:-len("__backward")]]
        ms = time_backward(bw, args.steps, args.warmup, torch, attn)
        tf = configs.backward_flops(bw) / (ms * 1e-3) / 1e12
        print(json.dumps({"metric": "backward TFLOP/s", "value": tf, "unit": "TFLOP/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "ms_spread": SPREAD.get(args.workload), "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                          "data": "synthetic (seeded generator, workloads/gen.py)",
                          "config": {"workload": args.workload},
                          "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                       "frac": tf / PEAK_BF16_TFLOPS, "traffic": None,
                                       "kernel": "bwd_pre + bwd_dq + bwd_dkdv"}}), flush=True)
        return 0
    if args.workload in configs.SOCKET_BY_NAME:
        sk = configs.SOCKET_BY_NAME[args.workload]
        ms = time_socket(sk, args.steps, args.warmup, torch, attn)
        gbs = configs.socket_bytes(sk) / (ms * 1e-3) / 1e9
        print(json.dumps({"metric": "SOCKET sparse decode HBM GB/s", "value": gbs, "unit": "GB/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "ms_spread": SPREAD.get(args.workload), "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                          "data": "synthetic (seeded generator, workloads/gen.py)",
                          "config": {"workload": sk.name},
                          "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                                       "kernel": "socket_score + socket_select + decode"}}), flush=True)
        return 0
    if args.workload in configs.STREAM_BY_NAME:
        # one streaming step (append + decode) on its own, for profiling
        sw = configs.STREAM_BY_NAME[args.workload]
        ms = time_stream(sw, args.steps, args.warmup, 3, torch, attn)
        r = stream_rate(sw, ms)
        print(json.dumps({"metric": "streaming decode HBM GB/s", "value": r["value"], "unit": r["unit"],
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "ms_spread": SPREAD.get(args.workload),
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                          "data": "synthetic (seeded generator, workloads/gen.py)",
                          "config": {"workload": sw.name},
                          "roofline": {"bound": "hbm", "achieved": r["value"], "peak": r["peak"], "unit": "GB/s",
                                       "frac": r["frac"], "traffic": None, "kernel": "decode_bf16"}}), flush=True)
        return 0
    w = configs.BY_NAME[args.workload]
    rot = args.rotate if args.rotate > 0 else default_rotation(w)
    ms, inp, first = time_workload(w, args.steps, args.warmup, rot, torch, attn, keep_first_output=True)
    r = rate(w, ms)
    kern = kernel_of(w)
    traffic = measured_traffic(kern, w.name)
    result = {
        "metric": METRIC,
        "value": r["value"],
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms, "ms_spread": SPREAD.get(args.workload),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded generator, workloads/gen.py)",
        "config": {"workload": w.name, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "L": w.L, "S": w.S, "E": w.E,
                   "mode": w.mode, "causal": w.causal, "window": w.window, "n_reg": w.n_reg, "sink": w.sink,
                   "decode": w.decode, "parallelism": "single GPU", "rotated_buffer_sets": rot},
        "roofline": {"bound": r["bound"], "achieved": r["value"], "peak": r["peak"], "unit": r["unit"],
                     "frac": r["frac"], "traffic": traffic, "kernel": kern,
                     "algorithmic_per_launch": configs.algorithmic_bytes(w) if w.decode
                     else configs.algorithmic_flops(w)},
    }
    mf = measured_mfma_busy(kern, w.name)
    if mf is not None:
        result["roofline"]["mfma_busy_counter"] = mf
    probes = None
    if not args.no_probe:
        log("[bench] probe peaks: bf16 GEMM and device copy")
        probes = probe_peaks(torch, attn)
        result["probe_peaks"] = probes
        attach_probe(result["roofline"], probes)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: timing the oracle on a row sample")
        base, parity = cpu_baseline(w, inp, first[0], first[1], args.cpu_seconds)
        result["cpu_baseline"] = base
        result["parity"] = parity
    del inp, first
    if args.extras == "all":
        extras = {}
        for x in configs.ALL + configs.EXTRA:
            if x.name == w.name:
                continue
            rot = default_rotation(x)
            xms, xinp, xfirst = time_workload(x, args.steps, args.warmup, rot, torch, attn,
                                              keep_first_output=not args.no_cpu_baseline)
            xr = rate(x, xms)
            xr["ms"] = xms
            xr["ms_spread"] = SPREAD.get(x.name)
            xr["kernel"] = kernel_of(x)
            xr["rotated_buffer_sets"] = rot
            xt = measured_traffic(kernel_of(x), x.name)
            if xt is not None:
                xr["traffic"] = xt
            xm = measured_mfma_busy(kernel_of(x), x.name)
            if xm is not None:
                xr["mfma_busy_counter"] = xm
            attach_probe(xr, probes)
            if not args.no_cpu_baseline:
                log(f"[bench] {x.name}: oracle on a row sample")
                xr["cpu_baseline"], xr["parity"] = cpu_baseline(x, xinp, xfirst[0], xfirst[1],
                                                                args.cpu_seconds_extra)
            del xinp, xfirst
            torch.cuda.empty_cache()
            extras[x.name] = xr
        for bw in configs.BACKWARD:
            xms = time_backward(bw, args.steps, args.warmup, torch, attn)
            torch.cuda.empty_cache()
            tf = configs.backward_flops(bw) / (xms * 1e-3) / 1e12
            extras[bw.name + "__backward"] = {
                "value": tf, "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
                "frac": tf / PEAK_BF16_TFLOPS, "ms": xms, "ms_spread": SPREAD.get(bw.name + "__backward"),
                "kernel": "bwd_dq + bwd_dkdv",
                "hbm_GBps": configs.backward_bytes(bw) / (xms * 1e-3) / 1e9,
                "algorithmic_per_step": configs.backward_flops(bw)}
            attach_probe(extras[bw.name + "__backward"], probes)
        for sk in configs.SOCKET_BY_NAME.values():
            xms = time_socket(sk, args.steps, args.warmup, torch, attn)
            torch.cuda.empty_cache()
            gbs = configs.socket_bytes(sk) / (xms * 1e-3) / 1e9
            dense = extras.get(sk.base.name, {}).get("ms")
            extras[sk.name] = {"value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
                               "frac": gbs / PEAK_HBM_GBS, "ms": xms, "ms_spread": SPREAD.get(sk.name),
                               "kernel": "socket_prob + socket_score + socket_select + decode (indexed)",
                               "speedup_vs_dense_decode": (dense / xms) if dense else None}
            attach_probe(extras[sk.name], probes)
        for sw in configs.STREAM_BY_NAME.values():
            xms = time_stream(sw, args.steps, args.warmup, 3, torch, attn)
            torch.cuda.empty_cache()
            xr = stream_rate(sw, xms)
            xr["ms"] = xms
            xr["ms_spread"] = SPREAD.get(sw.name)
            xr["kernel"] = "stream_append + decode_bf16"
            xr["rotated_buffer_sets"] = 3
            attach_probe(xr, probes)
            extras[sw.name] = xr
        result["extras"] = extras
        dec = extras.get(configs.C5.name)
        if dec is not None:
            # the metric's second half: long-context split-K decode against the HBM roofline
            result["decode"] = {"workload": configs.C5.name, "value": dec["value"], "unit": dec["unit"],
                                "peak": dec["peak"], "frac": dec["frac"], "ms": dec["ms"],
                                "probe_peak": dec.get("probe_peak"), "frac_of_probe": dec.get("frac_of_probe"),
                                "parity_pass": dec.get("parity", {}).get("pass")}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
