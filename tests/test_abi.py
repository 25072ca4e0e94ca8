"""The C ABI on the host: the library loads, exports every declared entry
point, sizes agree with the pages' worked examples and with the oracle, and
bad arguments are rejected before any GPU work.  CPU only (no kernel runs:
every call here fails validation or is a pure host function)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_expert_dispatch_amd as M
from sparse_expert_dispatch_amd import _native as N
from oracle import moe_oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_dispatch.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(N.LIB_PATH):
        pytest.fail(f"{N.LIB_PATH} not built (run python -m sparse_expert_dispatch_amd.build)")
    return N.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 29
    for name in names:
        assert hasattr(L, name), name
    assert sorted(N.EXPORTED) == names


def test_sizes_match_worked_examples_and_oracle(L):
    assert M.moe_ec_k(4096, 2.0, 64) == 128          # page 1 "Who picks whom"
    assert M.moe_ec_k(1024, 2.0, 8) == 256           # page 2 "A worked example"
    assert M.moe_tc_capacity(16384, 1, 128, 1.25) == 160
    assert M.moe_tc_capacity(256, 2, 8, 1.25) == 80
    rng = np.random.default_rng(0)
    for _ in range(2000):
        n, E, k = int(rng.integers(1, 20000)), int(rng.integers(1, 300)), int(rng.integers(1, 9))
        c = float(rng.choice([0.5, 1.0, 1.25, 2.0, 3.3]))
        assert M.moe_ec_k(n, c, E) == O.ec_k(n, c, E)
        assert M.moe_tc_capacity(n, k, E, c) == O.tc_capacity(n, k, E, c)
    assert M.moe_ec_k(0, 2.0, 8) == -1 and M.moe_tc_capacity(10, 0, 8, 1.0) == -1


def test_max_slots(L):
    cfg = N.make_cfg(256, 64, 8, 2, capacity=80)
    assert M.moe_max_slots(cfg) == 512
    cfg = N.make_cfg(256, 64, 8, 2, capacity=40)
    assert M.moe_max_slots(cfg) == 320
    assert M.moe_token_list_len(cfg) == 512
    cfg = N.make_cfg(4096, 2048, 64, 128, direction=N.MOE_EXPERT_CHOICE)
    assert M.moe_max_slots(cfg) == 8192
    assert M.moe_token_list_len(cfg) == 8192


FAKE = 0x10000   # a non-NULL, 16-byte aligned address that is never dereferenced


def _router(L, cfg, dtype=N.MOE_BF16, x=FAKE, ws=None, wsb=0, noise=None, noise_std=0.0):
    return L.moe_router(x, FAKE, dtype, None, noise, noise_std, ctypes.byref(cfg), FAKE, None, None, ws,
                        wsb, None)


@pytest.mark.parametrize("bad, status", [
    (dict(n=0), N.MOE_ERR_INVALID_ARG),
    (dict(k=9), N.MOE_ERR_INVALID_ARG),                       # k > E
    (dict(E=600, k=2), N.MOE_ERR_UNSUPPORTED),                 # beyond 512 experts
    (dict(n_group=3), N.MOE_ERR_INVALID_ARG),                  # E % n_group
    (dict(n_group=4, topk_group=5), N.MOE_ERR_INVALID_ARG),
    (dict(n_group=4, topk_group=1, k=3), N.MOE_ERR_INVALID_ARG),   # k > experts in kept groups
    (dict(capacity=-2), N.MOE_ERR_INVALID_ARG),
    (dict(score=7), N.MOE_ERR_INVALID_ARG),
    (dict(group_topm=0), N.MOE_ERR_INVALID_ARG),
    (dict(capacity_order=2), N.MOE_ERR_INVALID_ARG),
])
def test_config_validation(L, bad, status):
    kw = dict(n=256, d=64, E=8, k=2)
    kw.update(bad)
    n, d, E, k = kw.pop("n"), kw.pop("d"), kw.pop("E"), kw.pop("k")
    cfg = N.make_cfg(n, d, E, k, **kw)
    assert _router(L, cfg, N.MOE_F32) == status
    assert L.moe_last_error().decode() != ""


def test_expert_choice_validation(L):
    cfg = N.make_cfg(100, 64, 8, 101, direction=N.MOE_EXPERT_CHOICE)      # k > n
    assert _router(L, cfg, N.MOE_F32) == N.MOE_ERR_INVALID_ARG
    cfg = N.make_cfg(100, 64, 8, 10, direction=N.MOE_EXPERT_CHOICE, score=N.MOE_SIGMOID)
    assert _router(L, cfg, N.MOE_F32) == N.MOE_ERR_UNSUPPORTED


def test_routing_variant_validation(L):
    # sqrtsoftplus scores and rank-major capacity are token-choice options
    cfg = N.make_cfg(100, 64, 8, 10, direction=N.MOE_EXPERT_CHOICE, score=N.MOE_SQRTSOFTPLUS)
    assert _router(L, cfg, N.MOE_F32) == N.MOE_ERR_UNSUPPORTED
    cfg = N.make_cfg(100, 64, 8, 10, direction=N.MOE_EXPERT_CHOICE, capacity_order=N.MOE_RANK_MAJOR)
    assert _router(L, cfg, N.MOE_F32) == N.MOE_ERR_INVALID_ARG
    # noise needs a finite scale; without noise the scale is ignored
    cfg = N.make_cfg(256, 64, 8, 2, score=N.MOE_SQRTSOFTPLUS, capacity_order=N.MOE_RANK_MAJOR)
    assert _router(L, cfg, N.MOE_F32, noise=FAKE, noise_std=float("nan")) == N.MOE_ERR_INVALID_ARG
    assert _router(L, cfg, N.MOE_F32, noise=FAKE, noise_std=float("inf")) == N.MOE_ERR_INVALID_ARG
    # the bias update: token choice only, non-NULL buffers, finite gamma
    assert L.moe_update_bias(FAKE, ctypes.byref(cfg), 0.001, None, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_update_bias(FAKE, ctypes.byref(cfg), float("nan"), FAKE, None) == N.MOE_ERR_INVALID_ARG
    ec = N.make_cfg(100, 64, 8, 10, direction=N.MOE_EXPERT_CHOICE)
    assert L.moe_update_bias(FAKE, ctypes.byref(ec), 0.001, FAKE, None) == N.MOE_ERR_INVALID_ARG
    bad = N.make_cfg(256, 64, 8, 9)
    assert L.moe_update_bias(FAKE, ctypes.byref(bad), 0.001, FAKE, None) == N.MOE_ERR_INVALID_ARG


def test_null_pointers_and_unsupported_shapes(L):
    cfg = N.make_cfg(256, 64, 8, 2)
    assert _router(L, cfg, N.MOE_F32, x=None) == N.MOE_ERR_INVALID_ARG
    cfg = N.make_cfg(256, 128, 16, 2)                     # misaligned bf16 input
    assert _router(L, cfg, N.MOE_BF16, x=FAKE + 2) == N.MOE_ERR_INVALID_ARG
    # expert FFN: bf16 shapes and workspace
    st = L.moe_expert_ffn(FAKE, N.MOE_BF16, FAKE, 8, 100, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE,
                          FAKE, 1 << 30, None)
    assert st == N.MOE_ERR_UNSUPPORTED
    st = L.moe_expert_ffn(FAKE, N.MOE_BF16, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE,
                          FAKE, 16, None)
    assert st == N.MOE_ERR_WORKSPACE
    st = L.moe_expert_ffn(FAKE, N.MOE_BF16, None, 8, 128, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE,
                          FAKE, 1 << 30, None)
    assert st == N.MOE_ERR_INVALID_ARG


def test_packed_weight_validation(L):
    pack = L.moe_pack_expert_weights
    assert pack(None, 8, 128, 64, 0, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert pack(FAKE, 8, 128, 64, 0, FAKE, None) == N.MOE_ERR_INVALID_ARG          # aliased
    assert pack(FAKE, 8, 100, 64, 0, FAKE + 4096, None) == N.MOE_ERR_UNSUPPORTED   # rows % 32
    assert pack(FAKE, 8, 96, 64, 1, FAKE + 4096, None) == N.MOE_ERR_UNSUPPORTED    # gate/up: rows % 64
    assert pack(FAKE, 8, 128, 48, 0, FAKE + 4096, None) == N.MOE_ERR_UNSUPPORTED   # K % 64
    assert pack(FAKE, 8, 128, 64, 2, FAKE + 4096, None) == N.MOE_ERR_INVALID_ARG
    assert pack(FAKE + 8, 8, 128, 64, 0, FAKE + 4096, None) == N.MOE_ERR_INVALID_ARG   # misaligned
    ffn = L.moe_expert_ffn_packed
    assert ffn(None, 0, None, None, 8, 128, 128, N.MOE_GELU, None, None, 0, None, None, 0, None) == N.MOE_OK
    assert ffn(FAKE, 0, None, FAKE, 8, 100, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE, FAKE, 1 << 30, None) == \
        N.MOE_ERR_UNSUPPORTED
    assert ffn(FAKE, 0, None, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE, FAKE, 16, None) == \
        N.MOE_ERR_WORKSPACE
    assert ffn(FAKE, 0, None, None, 8, 128, 128, N.MOE_SWIGLU, FAKE, FAKE, 64, FAKE, FAKE, 1 << 30, None) == \
        N.MOE_ERR_INVALID_ARG
    assert ffn(FAKE, 0, None, FAKE, 8, 128, 128, 7, FAKE, FAKE, 64, FAKE, FAKE, 1 << 30, None) == \
        N.MOE_ERR_INVALID_ARG
    # the fused gather needs the row count of X
    assert ffn(FAKE, 0, FAKE, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE, FAKE, 1 << 30, None) == \
        N.MOE_ERR_INVALID_ARG
    up, down = L.moe_expert_up_packed, L.moe_expert_down_packed
    W = FAKE + 8192                                          # a workspace
    wsb = N.MOE_GEMM_WS_BYTES
    assert up(None, 0, None, None, 8, 128, 128, N.MOE_GELU, None, 0, None, None, 0, None) == N.MOE_OK
    assert down(None, None, 8, 128, 128, None, 0, None, None, 0, None) == N.MOE_OK
    assert up(FAKE, 0, None, FAKE, 8, 100, 128, N.MOE_GELU, FAKE, 64, FAKE + 4096, W, wsb, None) == \
        N.MOE_ERR_UNSUPPORTED
    assert up(FAKE, 0, FAKE, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, 64, FAKE + 4096, W, wsb, None) == \
        N.MOE_ERR_INVALID_ARG
    assert up(FAKE, 0, None, FAKE, 8, 128, 128, 3, FAKE, 64, FAKE + 4096, W, wsb, None) == N.MOE_ERR_INVALID_ARG
    assert up(FAKE, 0, None, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, 64, FAKE, W, wsb, None) == \
        N.MOE_ERR_INVALID_ARG                                                                     # H = X
    assert up(FAKE + 8, 0, None, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, 64, FAKE + 4096, W, wsb, None) == \
        N.MOE_ERR_INVALID_ARG                                                                     # misaligned
    assert up(FAKE, 0, None, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, 64, FAKE + 4096, W, wsb - 1, None) == \
        N.MOE_ERR_WORKSPACE
    assert up(FAKE, 0, None, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, 64, FAKE + 4096, None, wsb, None) == \
        N.MOE_ERR_WORKSPACE
    assert down(FAKE, None, 8, 128, 128, FAKE, 64, FAKE + 4096, W, wsb, None) == N.MOE_ERR_INVALID_ARG   # offsets
    assert down(FAKE, FAKE, 8, 128, 96, FAKE, 64, FAKE + 4096, W, wsb, None) == N.MOE_ERR_UNSUPPORTED    # f % 64
    assert down(FAKE, FAKE, 8, 128, 128, FAKE, 64, FAKE, W, wsb, None) == N.MOE_ERR_INVALID_ARG          # Y = H
    assert down(FAKE, FAKE, 8, 128, 128, FAKE, -1, FAKE + 4096, W, wsb, None) == N.MOE_ERR_INVALID_ARG
    assert down(FAKE, FAKE, 8, 128, 128, FAKE, 64, FAKE + 4096, W + 4, wsb, None) == \
        N.MOE_ERR_INVALID_ARG                                                                     # ws misaligned
    assert down(FAKE, FAKE, 8, 128, 128, FAKE, 64, FAKE + 4096, W, 16, None) == N.MOE_ERR_WORKSPACE


def test_noalloc_ffn_argument_checks(L):
    """The no-alloc FFN rejects what moe_expert_ffn_packed rejects, and shapes
    whose workspace exceeds its fixed array, before touching a device."""
    na = L.moe_expert_ffn_packed_noalloc
    assert na(None, 0, None, None, 8, 128, 128, N.MOE_GELU, None, None, 0, None, None) == N.MOE_OK
    assert na(FAKE, 0, None, FAKE, 8, 100, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE, None) == N.MOE_ERR_UNSUPPORTED
    assert na(FAKE, 0, None, None, 8, 128, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert na(FAKE, 0, None, FAKE, 8, 128, 128, 5, FAKE, FAKE, 64, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert na(FAKE, 0, FAKE, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert na(FAKE + 2, 0, None, FAKE, 8, 128, 128, N.MOE_GELU, FAKE, FAKE, 64, FAKE, None) == N.MOE_ERR_INVALID_ARG
    # M_max x f x 2 bytes beyond the 64 MiB array
    assert na(FAKE, 0, None, FAKE, 8, 128, 4096, N.MOE_GELU, FAKE, FAKE, 8193, FAKE, None) == N.MOE_ERR_WORKSPACE
    assert b"fixed" in L.moe_last_error()
    assert N.MOE_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_workspace_checks(L):
    cfg = N.make_cfg(4096, 2048, 64, 128, direction=N.MOE_EXPERT_CHOICE)
    need = M.moe_route_workspace_size(cfg)
    assert need >= 4096 * 64 * 4
    cm = N.RouteMapC(*([FAKE] * 8))
    assert L.moe_build_map(FAKE, FAKE, ctypes.byref(cfg), ctypes.byref(cm), FAKE, 8, None) == \
        N.MOE_ERR_WORKSPACE
    cm_bad = N.RouteMapC(*([FAKE] * 7 + [0]))
    assert L.moe_build_map(FAKE, FAKE, ctypes.byref(cfg), ctypes.byref(cm_bad), FAKE, need, None) == \
        N.MOE_ERR_INVALID_ARG
    # select without precomputed scores needs the transpose workspace
    assert L.moe_select(FAKE, None, None, ctypes.byref(cfg), FAKE, FAKE, FAKE, 8, None) == \
        N.MOE_ERR_WORKSPACE
    assert L.moe_balance_stats(FAKE, ctypes.byref(cm), ctypes.byref(cfg), 0.01, 0.001, FAKE, None,
                               FAKE, 4, None) == N.MOE_ERR_WORKSPACE
    # combine output must not alias an input
    assert L.moe_combine(FAKE, N.MOE_BF16, ctypes.byref(cm), 16, 64, None, None, FAKE, None) == \
        N.MOE_ERR_INVALID_ARG


def test_status_strings(L):
    assert M.moe_status_string(0) == "ok"
    assert M.moe_status_string(3) == "workspace too small"
    assert M.moe_status_string(99) == "unknown status"


def test_python_binding_refuses_cpu_tensors(L):
    import torch
    cfg = N.make_cfg(16, 64, 8, 2)
    x = torch.zeros(16, 64)
    with pytest.raises(ValueError):
        M.moe_router(x, torch.zeros(64, 8), None, cfg, torch.zeros(16, 8))


def test_backward_validation(L):
    """The backward entry points reject bad arguments on the host."""
    cfg = N.make_cfg(256, 128, 8, 2)
    cm = N.RouteMapC(*([FAKE] * 8))
    cmb = ctypes.byref(cm)
    # combine backward: aliasing, dtype, M_max = 0 is a no-op
    assert L.moe_combine_backward(FAKE, FAKE + 4096, N.MOE_BF16, 256, 128, cmb, 512, FAKE, FAKE, None) == \
        N.MOE_ERR_INVALID_ARG
    assert L.moe_combine_backward(FAKE, FAKE + 4096, 5, 256, 128, cmb, 512, FAKE + 8192, FAKE, None) == \
        N.MOE_ERR_INVALID_ARG
    assert L.moe_combine_backward(None, None, N.MOE_BF16, 256, 128, cmb, 0, None, None, None) == N.MOE_OK
    assert L.moe_combine_backward(FAKE + 2, FAKE + 4096, N.MOE_BF16, 256, 128, cmb, 512, FAKE + 8192, FAKE,
                                  None) == N.MOE_ERR_INVALID_ARG                        # misaligned bf16
    # expert FFN backward: workspace, activation, null weights
    need = M.moe_ffn_backward_workspace_size(512, 8, 128, 64, N.MOE_SWIGLU, N.MOE_BF16)
    assert need >= 512 * (128 + 64 + 128) * 2
    ffn = L.moe_expert_ffn_backward
    assert ffn(FAKE, N.MOE_BF16, FAKE, 8, 128, 64, N.MOE_SWIGLU, FAKE, FAKE, FAKE, 512, FAKE, FAKE, FAKE,
               FAKE, 16, None) == N.MOE_ERR_WORKSPACE
    assert ffn(FAKE, N.MOE_BF16, FAKE, 8, 128, 64, 3, FAKE, FAKE, FAKE, 512, FAKE, FAKE, FAKE, FAKE, need,
               None) == N.MOE_ERR_INVALID_ARG
    assert ffn(FAKE, N.MOE_BF16, FAKE, 8, 128, 64, N.MOE_GELU, None, FAKE, FAKE, 512, FAKE, FAKE, FAKE, FAKE,
               need, None) == N.MOE_ERR_INVALID_ARG
    assert ffn(FAKE, N.MOE_BF16, FAKE, 1024, 128, 64, N.MOE_GELU, FAKE, FAKE, FAKE, 512, FAKE, FAKE, FAKE,
               FAKE, need, None) == N.MOE_ERR_UNSUPPORTED                               # E > 512
    # gate backward: token choice needs sel_idx; the map must be complete
    assert L.moe_gate_backward(FAKE, None, FAKE, ctypes.byref(cfg), cmb, 0.01, 0.001, FAKE, None) == \
        N.MOE_ERR_INVALID_ARG
    cm_bad = N.RouteMapC(*([FAKE] * 7 + [0]))
    assert L.moe_gate_backward(FAKE, FAKE, FAKE, ctypes.byref(cfg), ctypes.byref(cm_bad), 0.01, 0.001, FAKE,
                               None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_gate_backward(FAKE, FAKE, FAKE, ctypes.byref(cfg), cmb, float("nan"), 0.001, FAKE, None) == \
        N.MOE_ERR_INVALID_ARG
    # router backward: workspace and aliasing
    rneed = M.moe_router_backward_workspace_size(cfg, N.MOE_BF16)
    assert rneed >= 256 * 8 * 2
    assert L.moe_router_backward(FAKE, FAKE, N.MOE_BF16, FAKE, ctypes.byref(cfg), None, FAKE + 4096, FAKE, FAKE,
                                 FAKE, 8, None) == N.MOE_ERR_WORKSPACE
    assert L.moe_router_backward(FAKE, FAKE, N.MOE_BF16, FAKE, ctypes.byref(cfg), None, FAKE, FAKE, FAKE, FAKE,
                                 rneed, None) == N.MOE_ERR_INVALID_ARG                  # dX aliases X
    # dispatch backward: output must not alias an input
    assert L.moe_dispatch_backward(FAKE, N.MOE_BF16, cmb, 256, 128, FAKE + 4096, None, FAKE + 4096, None) == \
        N.MOE_ERR_INVALID_ARG
