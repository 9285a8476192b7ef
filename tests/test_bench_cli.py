"""bench.py's command line on the host: more than one GPU is refused with a
message before anything touches a GPU; the workloads it names exist, with
the decode variants on the Mixtral-shaped weights and tokens."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_workloads_named_in_the_bench_exist():
    from moe_synth.configs import CONFIGS
    for name in ("tiny", "mixtral", "decode", "decode_fp8", "decode_int8", "decode_int4",
                 "fine_grained", "fine_grained_fp8", "fine_grained_int8", "fine_grained_int4",
                 "capacity_skew"):
        assert name in CONFIGS
    # the decode variants share the Mixtral-shaped weights and tokens
    for name in ("decode", "decode_fp8", "decode_int8", "decode_int4"):
        c = CONFIGS[name]
        assert (c.T, c.d, c.E, c.k, c.d_ff) == (64, 4096, 8, 2, 14336)
        assert c.w_from == "mixtral" and c.x_from == "mixtral"
