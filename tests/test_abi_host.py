"""Host-side checks of the libmoe C ABI (no GPU): the library loads, exports every entry
point include/moe.h declares, and rejects bad arguments before anything is enqueued.
The invalid-argument calls below return during host validation, before any HIP call,
so they are safe without a device (pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.library_path()):
        from sparse_mixture_experts_gemm_amd import build
        build.build()
    return moe.lib()


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ["moe_route", "moe_select", "moe_permute", "moe_grouped_gemm", "moe_combine",
                 "moe_forward", "moe_workspace_size", "moe_status_string", "moe_last_hip_error"]:
        assert name in fns
    assert sorted(moe.EXPORTED_SYMBOLS) == fns


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", moe.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    assert moe.status_string(0) == "ok"
    assert "workspace" in moe.status_string(3)
    assert moe.status_string(99) == "unknown status"
    assert lib.moe_last_hip_error() == 0


def cfg(**kw):
    base = dict(T=4096, d=2048, E=64, k=6, G=8, Gk=4, n_g=1, S=4, I=1536)
    base.update(kw)
    T, d, E, k, I = base.pop("T"), base.pop("d"), base.pop("E"), base.pop("k"), base.pop("I")
    return moe.make_config(T, d, E, k, I=I, **base)


def test_workspace_size_is_the_sum_of_the_stages(lib):
    n = moe.workspace_size(cfg())
    T, k, d, I, S = 4096, 6, 2048, 1536, 4
    inter = T * k * I * 2 + T * S * I * 2 + T * k * d * 2 + T * d * 2
    assert inter <= n <= inter + 8 * 1024 * 1024
    assert moe.workspace_size(cfg(T=0)) < 64 * 1024
    assert moe.workspace_size(cfg(T=64)) < moe.workspace_size(cfg(T=128))


@pytest.mark.parametrize("bad,status", [
    (dict(k=0), 1), (dict(k=65, E=64), 1), (dict(E=60, G=8), 1), (dict(Gk=9), 1),
    (dict(k=17, Gk=2), 1), (dict(n_g=3), 1), (dict(E=64, G=64, Gk=6, n_g=2), 1),
    (dict(T=-1), 1), (dict(d=0), 1), (dict(E=128, G=8, k=6), 2), (dict(d=2004), 2),
    (dict(I=1004), 2), (dict(weight_dtype="e4m3", d=2056), 2),   # 8 | d but not 16 (e4m3)
    (dict(weight_dtype="e4m3", I=1544), 2), (dict(act_dtype="f32", weight_dtype="f32", d=40), 2),
    (dict(act_dtype="f32", weight_dtype="bf16"), 2),
    (dict(act_dtype="bf16", weight_dtype="f32"), 2),
    (dict(capacity_factor=float("nan")), 1),
    (dict(fp8_act=True), 2),                       # e4m3 activations need e4m3 weights
    (dict(fp8_act=True, weight_dtype="e4m3", d=192), 2),   # ... and 128-byte K-slices
    (dict(fp8_act=True, weight_dtype="e4m3", I=1552), 2),  # ... and 64-wide output tiles
    (dict(pre_norm=True, norm_eps=float("nan")), 1), (dict(norm_eps=-1e-6), 1),
    # the stacked shared experts' weights past 2^31 - 1 elements
    (dict(T=64, E=8, G=8, Gk=2, k=2, S=64, d=4096, I=8192), 2),
])
def test_invalid_configs_are_rejected_on_the_host(lib, bad, status):
    c = cfg(**bad)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == status
    fake = 4096   # never dereferenced: validation fails first
    assert lib.moe_route(ctypes.byref(c), fake, fake, None, None, None, fake, fake, None) == status
    assert lib.moe_select(ctypes.byref(c), fake, None, fake, fake, None) == status
    assert lib.moe_load_stats(ctypes.byref(c), fake, fake, 1.0, fake, fake, fake, fake, 1 << 20,
                              None) == status
    with pytest.raises(moe.MoeError):
        moe.workspace_size(c)


def test_prenorm_config_and_route_arguments_are_checked_on_the_host(lib):
    c = cfg(T=64, pre_norm=True, residual=True)
    plain = moe.workspace_size(cfg(T=64))
    assert moe.workspace_size(c) == plain + 64 * 2048 * 2       # the normalised rows
    for field in ("pre_norm", "residual"):
        bad = cfg(T=64)
        setattr(bad, field, 2)
        n = ctypes.c_size_t(0)
        assert lib.moe_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == 1
    fake = 4096
    # moe_rmsnorm_route(cfg, x, gamma, router, logit_bias, select_bias, x_norm, scores, idx, w)
    assert lib.moe_rmsnorm_route(ctypes.byref(c), fake, None, fake, None, None, fake + 4096, None,
                                 fake, fake, None) == 1                      # no gain
    assert lib.moe_rmsnorm_route(ctypes.byref(c), fake, fake, fake, None, None, None, None,
                                 fake, fake, None) == 1                      # no output rows
    assert lib.moe_rmsnorm_route(ctypes.byref(c), fake, fake, fake, None, None, fake, None,
                                 fake, fake, None) == 1                      # x_norm aliases x
    assert lib.moe_rmsnorm_route(ctypes.byref(c), fake, fake + 4, fake, None, None, fake + 4096,
                                 None, fake, fake, None) == 2                # misaligned gain
    c0 = cfg(T=0, pre_norm=True)
    assert lib.moe_rmsnorm_route(ctypes.byref(c0), None, None, None, None, None, None, None,
                                 None, None, None) == 0
    # the forward of a pre-norm layer needs the gain
    w = moe.Weights(router=fake, w_gate=fake, w_up=fake, w_down=fake, sh_gate=fake, sh_up=fake,
                    sh_down=fake)
    need = moe.workspace_size(c)
    assert lib.moe_forward(ctypes.byref(c), ctypes.byref(w.c), fake, fake, fake, need, None) == 1


def test_backward_arguments_are_checked_on_the_host(lib):
    c = cfg(T=64)
    n = moe.backward_workspace_size(c)
    assert n > moe.workspace_size(c)
    fake = 4096
    w = moe.Weights(router=fake, w_gate=fake, w_up=fake, w_down=fake, sh_gate=fake, sh_up=fake,
                    sh_down=fake)
    fwd = moe.workspace_size(c)
    g = moe._GradsC(dx=fake)
    call = lambda cc, ww, gg, fb=fwd, nb=n, x=fake: lib.moe_backward(
        ctypes.byref(cc), ctypes.byref(ww.c), x, fake, fake, fb, ctypes.byref(gg), fake, nb, None)
    assert call(c, w, moe._GradsC()) == 1                  # dx is required
    assert call(c, w, g, x=None) == 1
    assert call(c, w, g, fb=fwd - 1) == 3                   # forward workspace too small
    assert call(c, w, g, nb=n - 1) == 3                     # backward workspace too small
    assert call(c, w, g, x=fake + 2) == 2                   # misaligned
    for bad, status in [(dict(weight_dtype="e4m3"), 2), (dict(act_dtype="f32", weight_dtype="f32"), 2),
                        (dict(pre_norm=True), 2), (dict(route_scale=0.0), 1),
                        (dict(d=2000), 2), (dict(I=1000), 2)]:   # the backward's 64-grid
        cb = cfg(T=64, **bad)
        nn = ctypes.c_size_t(0)
        assert lib.moe_backward_workspace_size(ctypes.byref(cb), ctypes.byref(nn)) == status
        assert call(cb, w, g) == status
    c0 = cfg(T=0)
    assert lib.moe_backward(ctypes.byref(c0), ctypes.byref(w.c), None, None, None, 0,
                            ctypes.byref(g), None, 0, None) == 0


def test_null_and_workspace_errors_are_reported_before_launch(lib):
    c = cfg(T=64)
    fake = 4096
    w = moe.Weights(router=fake, w_gate=fake, w_up=fake, w_down=fake, sh_gate=fake, sh_up=fake,
                    sh_down=fake)
    need = moe.workspace_size(c)
    # workspace too small
    assert lib.moe_forward(ctypes.byref(c), ctypes.byref(w.c), fake, fake, fake, need - 1, None) == 3
    assert lib.moe_forward(ctypes.byref(c), ctypes.byref(w.c), fake, fake, None, need, None) == 3
    # null x / out / weights
    assert lib.moe_forward(ctypes.byref(c), ctypes.byref(w.c), None, fake, fake, need, None) == 1
    assert lib.moe_forward(ctypes.byref(c), None, fake, fake, fake, need, None) == 1
    w_missing = moe.Weights(router=fake, w_gate=fake, w_down=fake, sh_gate=fake, sh_up=fake,
                            sh_down=fake)
    assert lib.moe_forward(ctypes.byref(c), ctypes.byref(w_missing.c), fake, fake, fake, need,
                           None) == 1
    # misaligned pointer
    assert lib.moe_forward(ctypes.byref(c), ctypes.byref(w.c), fake + 2, fake, fake, need, None) == 2
    # permute: workspace and optional weight pair
    assert lib.moe_permute(ctypes.byref(c), fake, None, fake, fake, fake, fake, None, None, 0, None) == 3
    assert lib.moe_permute(ctypes.byref(c), fake, fake, fake, fake, fake, fake, None, fake, 1 << 20,
                           None) == 1
    # grouped gemm: routed set needs offsets; shared set needs S > 0; bad stage
    assert lib.moe_grouped_gemm(ctypes.byref(c), 0, 0, fake, None, None, 10, ctypes.byref(w.c), None,
                                fake, None, 0, None) == 1
    c0 = cfg(T=64, S=0)
    assert lib.moe_grouped_gemm(ctypes.byref(c0), 0, 1, fake, None, None, 10, ctypes.byref(w.c), None,
                                fake, None, 0, None) == 1
    assert lib.moe_grouped_gemm(ctypes.byref(c), 7, 0, fake, None, fake, 10, ctypes.byref(w.c), None,
                                fake, None, 0, None) == 1
    # combine: null y
    assert lib.moe_combine(ctypes.byref(c), None, fake, None, fake, None) == 1
    # quantize: null output, columns not a multiple of 8, fp32 activations
    assert lib.moe_quantize_rows(ctypes.byref(c), fake, 4, 64, None, fake, None) == 1
    assert lib.moe_quantize_rows(ctypes.byref(c), fake, 4, 60, fake, fake, None) == 2
    c32 = moe.make_config(64, 64, 8, 2, I=64, act_dtype="f32", weight_dtype="f32")
    assert lib.moe_quantize_rows(ctypes.byref(c32), fake, 4, 64, fake, fake, None) == 2
    # grouped gemm with e4m3 activations: the up stage needs the row scales
    ca8 = cfg(T=64, weight_dtype="e4m3", fp8_act=True)
    assert lib.moe_grouped_gemm(ctypes.byref(ca8), 0, 1, fake, None, None, 10, ctypes.byref(w.c),
                                None, fake, None, 0, None) == 1
    # load statistics: null outputs, missing workspace, non-finite alpha
    assert lib.moe_load_stats(ctypes.byref(c), fake, fake, 1.0, None, fake, fake, fake, 1 << 20,
                              None) == 1
    assert lib.moe_load_stats(ctypes.byref(c), fake, fake, 1.0, fake, fake, fake, None, 0, None) == 3
    assert lib.moe_load_stats(ctypes.byref(c), fake, fake, float("inf"), fake, fake, fake, fake,
                              1 << 20, None) == 1


def test_zero_tokens_is_a_no_op(lib):
    c = cfg(T=0)
    fake = 4096
    w = moe.Weights(router=fake, w_gate=fake, w_up=fake, w_down=fake, sh_gate=fake, sh_up=fake,
                    sh_down=fake)
    assert lib.moe_route(ctypes.byref(c), None, None, None, None, None, None, None, None) == 0
    assert lib.moe_load_stats(ctypes.byref(c), None, None, 1.0, None, None, None, None, 0, None) == 0
    assert lib.moe_forward(ctypes.byref(c), ctypes.byref(w.c), None, None, None, 0, None) == 0
    assert lib.moe_combine(ctypes.byref(c), None, None, None, None, None) == 0
    assert lib.moe_grouped_gemm(ctypes.byref(c), 0, 0, None, None, None, 0, ctypes.byref(w.c), None,
                                None, None, 0, None) == 0


def test_product_path_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_LIB", None)
    monkeypatch.setattr(moe, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(moe.LibraryMissing):
        moe.workspace_size(cfg())


@pytest.mark.parametrize("over,stage,expert_set,rows,path", [
    # the FusionLLM layer at 4096 tokens: every stage on the tiled MFMA kernel
    (dict(), moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, 4096 * 6, moe.MOE_GEMM_PATH_TILED),
    (dict(), moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_ROUTED, 4096 * 6, moe.MOE_GEMM_PATH_TILED),
    (dict(), moe.MOE_STAGE_UP, moe.MOE_EXPERTS_SHARED, 4096, moe.MOE_GEMM_PATH_TILED),
    (dict(), moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_SHARED, 4096, moe.MOE_GEMM_PATH_TILED),
    (dict(weight_dtype="e4m3"), moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, 16384 * 6,
     moe.MOE_GEMM_PATH_TILED),
    # 64 tokens: weight streaming
    (dict(T=64), moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, 64 * 6, moe.MOE_GEMM_PATH_DECODE),
    (dict(T=64), moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_SHARED, 64, moe.MOE_GEMM_PATH_DECODE),
    # off the 64-element grid: the tail kernel, for either stage
    (dict(d=200, I=136), moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, 4096 * 6, moe.MOE_GEMM_PATH_TAIL),
    (dict(d=2048, I=136), moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_SHARED, 4096, moe.MOE_GEMM_PATH_TAIL),
    (dict(d=208, I=144, weight_dtype="e4m3"), moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_ROUTED, 64 * 6,
     moe.MOE_GEMM_PATH_TAIL),
    (dict(act_dtype="f32", weight_dtype="f32"), moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, 100,
     moe.MOE_GEMM_PATH_F32),
    (dict(weight_dtype="e4m3", fp8_act=True), moe.MOE_STAGE_UP, moe.MOE_EXPERTS_ROUTED, 100,
     moe.MOE_GEMM_PATH_FP8_ACT),
    (dict(weight_dtype="e4m3", fp8_act=True), moe.MOE_STAGE_DOWN, moe.MOE_EXPERTS_ROUTED, 4096 * 6,
     moe.MOE_GEMM_PATH_TILED),
])
def test_gemm_kernel_path(lib, over, stage, expert_set, rows, path):
    assert moe.gemm_kernel_path(cfg(**over), stage, expert_set, rows) == path


def test_gemm_kernel_path_rejects_bad_arguments(lib):
    p = ctypes.c_int32(-1)
    assert lib.moe_gemm_kernel_path(ctypes.byref(cfg()), 0, 0, 10, None) == 1
    assert lib.moe_gemm_kernel_path(ctypes.byref(cfg()), 2, 0, 10, ctypes.byref(p)) == 1
    assert lib.moe_gemm_kernel_path(ctypes.byref(cfg(S=0)), 0, 1, 10, ctypes.byref(p)) == 1
    assert lib.moe_gemm_kernel_path(ctypes.byref(cfg(d=2004)), 0, 0, 10, ctypes.byref(p)) == 2


def test_random_test_layers_are_inside_the_contract(lib):
    """The seeded random layers of the GPU sweeps are configurations the library accepts
    (host-side validation only), so every GPU case exercises a kernel, not an error path."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from test_gpu_parity import random_shape
    from test_gpu_backward import random_backward_shape
    from _dev import config
    for seed in range(96):
        moe.workspace_size(config(random_shape(seed)))
    for seed in range(32):
        moe.backward_workspace_size(config(random_backward_shape(seed)))
