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
