"""Host-side logic of bench.py (no GPU): the one-GPU guard, the source digest that ties a
profile's traffic figure to the kernel sources, and the algorithmic FLOP count."""
import os

import bench
import workloads as W


def test_more_than_one_gpu_is_refused_before_any_device_work(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_source_digest_is_deterministic_and_covers_every_source():
    a = bench.kernel_source_digest()
    assert a == bench.kernel_source_digest() and len(a) == 64
    assert bench.kernel_source_digest(bench.DECODE_SOURCES) != a
    for name in bench.GEMM_SOURCES + bench.DECODE_SOURCES:
        assert os.path.exists(os.path.join(bench.ROOT, "sparse_mixture_experts_gemm_amd", "csrc", name))


def test_missing_profile_gives_no_traffic_figure():
    assert bench.profiled_traffic("no_such_profile.txt") is None


def test_stage_flops_count_one_multiply_add_per_weight_and_token():
    # every routed slot and every shared expert multiplies its token row by each expert
    # matrix once: SwiGLU has three d x I matrices, two of them in the up projection
    s = W.SHAPES["fusionllm_bf16"]
    f = bench.stage_flops(s, s.T)
    per_token_matrix = 2 * s.d * s.I
    assert f["up_routed"] + f["down_routed"] == s.T * s.k * 3 * per_token_matrix
    assert f["up_shared"] + f["down_shared"] == s.T * s.S * 3 * per_token_matrix
    assert f["route"] == 2 * s.T * s.d * s.E
    r = W.SHAPES["fp8_relu2"]
    g = bench.stage_flops(r, r.T)
    assert g["up_routed"] == g["down_routed"] == r.T * r.k * 2 * r.d * r.I
