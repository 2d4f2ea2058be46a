"""bench.py's command-line contract on a host without a GPU: more than one GPU
is refused with a message and no JSON line, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    r = _run(["--steps", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE=4" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_every_workload():
    r = _run(["--help"])
    assert r.returncode == 0
    for name in ("dot_causal_bf16_4x16x2048x128", "decode_splitk_sink_bf16_8x32to8x131072x128",
                 "stream_sink4_win4092_bf16_8x32to8x128_pos100000", "socket_decode_sink_bf16_8x32to8x131072x128_k3972",
                 "rbf_causal_reg4_bf16_2x16x8192x64__backward"):
        assert name in r.stdout


def test_probe_fraction_follows_the_entry_bound():
    sys.path.insert(0, ROOT)
    import bench
    probes = {"bf16_gemm": {"value": 2000.0, "unit": "TFLOP/s"}, "hbm_copy": {"value": 4000.0, "unit": "GB/s"},
              "hbm_read": {"value": 5000.0, "unit": "GB/s"}}
    mfma = {"bound": "mfma", "unit": "TFLOP/s", "achieved": 500.0, "value": 1.0}
    bench.attach_probe(mfma, probes)
    assert mfma["probe_peak"] == 2000.0 and abs(mfma["frac_of_probe"] - 0.25) < 1e-12
    hbm = {"bound": "hbm", "unit": "GB/s", "value": 4000.0}
    bench.attach_probe(hbm, probes)
    assert abs(hbm["frac_of_probe"] - 0.8) < 1e-12
    alu = {"bound": "alu", "unit": "TFLOP/s", "value": 1.0}
    bench.attach_probe(alu, probes)
    assert "probe_peak" not in alu
    mixed = {"bound": "hbm", "unit": "TFLOP/s", "value": 1.0}
    bench.attach_probe(mixed, probes)
    assert "probe_peak" not in mixed
    none = {"bound": "mfma", "unit": "TFLOP/s", "value": 1.0}
    bench.attach_probe(none, None)
    assert "probe_peak" not in none


def test_probe_peaks_runs_on_small_sizes():
    """The probe leg's torch calls, on the CPU with tiny sizes and a stand-in for the
    GPU's events and streams (the real leg runs the same calls on the GPU)."""
    import types
    import torch
    sys.path.insert(0, ROOT)
    import bench

    class Event:
        def __init__(self, enable_timing=True):
            pass

        def record(self, stream=None):
            pass

        def elapsed_time(self, other):
            return 1.0

    cuda = types.SimpleNamespace(Event=Event, synchronize=lambda: None, current_stream=lambda dev=None: None,
                                 empty_cache=lambda: None)
    shim = types.SimpleNamespace(**{k: getattr(torch, k) for k in dir(torch) if not k.startswith("__")})
    shim.cuda = cuda
    saved = bench.WARM_MS
    bench.WARM_MS = 0.0
    # the library's probes stand in as host-side no-ops (they need a GPU)
    probes = types.SimpleNamespace(probe_read=lambda src, sink=None: torch.zeros(4, dtype=torch.int32),
                                   probe_copy=lambda src, dst: None)
    try:
        out = bench.probe_peaks(shim, probes, n=32, nbytes=1 << 16, device="cpu")
    finally:
        bench.WARM_MS = saved
    assert set(out) == {"bf16_gemm", "hbm_copy", "hbm_read", "hbm_read_kernel", "hbm_copy_kernel"}
    assert all(v["value"] > 0 for v in out.values())
