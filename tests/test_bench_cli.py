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


def test_roofline_floors_of_the_workloads():
    """The binding floors bench.py reports against: the Mixtral-shaped layer's
    2.886e12 expert FLOPs at 2.5 PFLOP/s (1.155 ms, MFMA-bound); the
    fine-grained layer's 257 experts' bf16 weights (22.64 GB) at 8 TB/s
    (2.83 ms, HBM-bound) against 1.30 ms of MFMA time; the same in fp8 codes
    with their scales (11.32 GB, 1.42 ms)."""
    import bench
    from moe_synth.configs import CONFIGS
    f = bench.roofline_floor(CONFIGS["mixtral"], [1024] * 8, 8192)
    assert f["bound"] == "mfma" and abs(f["floor_ms"] - 1.1545) < 1e-3
    assert f["touched_experts"] == 8
    f = bench.roofline_floor(CONFIGS["fine_grained"], [128] * 256, 32768)
    assert f["bound"] == "hbm" and abs(f["mfma_floor_ms"] - 1.2984) < 1e-3
    assert abs(bench.weight_bytes(CONFIGS["fine_grained"], 257) - 22.64e9) < 0.01e9
    assert 2.83 < f["hbm_floor_ms"] < 2.86
    f8 = bench.roofline_floor(CONFIGS["fine_grained_fp8"], [128] * 256, 32768)
    assert 1.41 < f8["hbm_floor_ms"] < 1.45 and f8["bound"] == "hbm"
    # an expert the step never touched costs no weight bytes
    f = bench.roofline_floor(CONFIGS["capacity_skew"], [640] * 30 + [0] * 34, 640 * 30)
    assert f["touched_experts"] == 30


def test_gemm_kernel_named_for_each_workload():
    """The expert GEMM kernel bench.py names: the ping-pong kernel at the
    Mixtral shape (1024 rows per expert) and for the bf16 256-expert layer
    (128 rows); for its fp8 variant (128 rows, under the 256-row threshold)
    the four-wave kernel in the gate/up projection and the ping-pong kernel's
    128 x 512 tiles in the down projection; the four-wave kernel for int4,
    decode-sized tiles at 16 rows."""
    import bench
    from moe_synth.configs import CONFIGS
    assert bench.gemm_kernel(CONFIGS["mixtral"], -1) == "grouped_gemm_pp_kernel"
    assert bench.gemm_kernel(CONFIGS["fine_grained"], -1) == "grouped_gemm_pp_kernel"
    assert bench.gemm_kernel(CONFIGS["fine_grained_fp8"], -1) == "grouped_gemm_dma_kernel"
    assert bench.gemm_kernel(CONFIGS["fine_grained_fp8"], -1, "down") == \
        "grouped_gemm_pp_kernel (128 x 512 tiles)"
    assert bench.gemm_kernel(CONFIGS["fine_grained_int4"], -1) == "grouped_gemm_dma_kernel"
    assert bench.gemm_kernel(CONFIGS["decode"], -1).startswith("grouped_gemm_dma_kernel (decode")
    c = CONFIGS["capacity_skew"]
    assert bench.gemm_kernel(c, 640) == "grouped_gemm_pp_kernel"


def test_gate_up_bytes_of_the_decode_step():
    """The decode step's gate/up launch moves W1 and W3 of the 8 touched
    experts (8 * 2 * 4096 * 14336 bf16 = 1.879 GB), the 128 gathered x rows
    and the 128 hidden rows it writes; fp8 codes halve the weights and add
    one fp32 scale per 128 rows."""
    import bench
    from moe_synth.configs import CONFIGS
    c = CONFIGS["decode"]
    w = 8 * 2 * 4096 * 14336 * 2
    assert bench.gate_up_bytes(c, [16] * 8) == w + 128 * 4096 * 2 + 128 * 14336 * 2
    assert bench.gate_up_bytes(c, [32] * 4 + [0] * 4) == w // 2 + 128 * 4096 * 2 + 128 * 14336 * 2
    f = CONFIGS["decode_fp8"]
    assert bench.gate_up_bytes(f, [16] * 8) == w // 2 + 8 * 2 * 112 * 4 + 128 * 4096 * 2 + 128 * 14336 * 2
