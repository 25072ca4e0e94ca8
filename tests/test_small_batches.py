"""Decode-shaped batches: a handful of tokens per layer call.

Token choice at n = 1 ... 256 (each expert sees a few rows, the grouped GEMM
streams the touched experts' weights for almost no arithmetic), and the
degenerate expert choice of a batch too small for any expert to take a
token: k = n c / E rounds to 0 (page 1 "Token choice vs expert choice
routing", section "Who picks whom"; page 2 "Expert choice routing",
section "The math"), so every token rides the residual (plus the shared
expert)."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_expert_dispatch_amd import _native as N
from sparse_expert_dispatch_amd import workloads as W

FAKE = 0x10000


def _ec_tiny(n):
    return W.SMALL_CONFIGS[2].scaled(f"ec_n{n}", n=n)


# ---------------------------------------------------------------- oracle (CPU)

def test_expert_choice_with_no_slot_is_the_residual():
    for n in (1, 3):
        cfg = _ec_tiny(n)
        assert O.ec_k(cfg.n, cfg.c, cfg.E) == 0
        inp = W.gen_inputs(cfg)
        r = O.forward(cfg, inp)
        assert r["map"]["n_kept"] == 0 and r["sel_idx"].shape == (cfg.E, 0)
        assert (r["map"]["token_offset"] == 0).all()
        x = inp["x"].astype(np.uint32) << np.uint32(16)
        assert np.array_equal(r["out"], x.view(np.float32).astype(np.float64))     # residual only
        st, hist = r["stats"], r["hist"]
        assert st[0] == 0.0 and st[2] == 0.0 and st[4] == 0 and st[6] == n
        assert hist[0] == n and hist[1:].sum() == 0


def test_expert_choice_first_slot_appears_at_half_a_token():
    # k = round(n c / E): the first token per expert appears once n c / E >= 1/2
    E, c = 16, 2.0
    ks = [O.ec_k(n, c, E) for n in range(1, 13)]
    assert ks[:3] == [0, 0, 0] and ks[3] == 1 and ks[11] == 2      # n = 4 gives 0.5 -> 1


# ---------------------------------------------------------------- ABI (CPU, no device work)

def test_abi_zero_slot_paths_return_before_touching_the_device():
    L = N.lib()
    ec0 = N.make_cfg(3, 256, 16, 0, direction=N.MOE_EXPERT_CHOICE)
    assert L.moe_max_slots(ctypes.byref(ec0)) == 0
    assert L.moe_token_list_len(ctypes.byref(ec0)) == 0
    assert L.moe_select(FAKE, None, None, ctypes.byref(ec0), None, None, None, 0, None) == N.MOE_OK
    assert L.moe_dispatch(FAKE, N.MOE_BF16, 3, 256, None, 0, None, None) == N.MOE_OK
    assert L.moe_expert_ffn(None, N.MOE_BF16, None, 16, 256, 512, N.MOE_GELU, None, None, 0, None, None,
                            0, None) == N.MOE_OK
    size = ctypes.c_size_t()
    assert L.moe_ffn_workspace_size(0, 16, 256, 512, N.MOE_GELU, N.MOE_BF16, ctypes.byref(size)) == N.MOE_OK
    assert size.value == 0
    tc0 = N.make_cfg(3, 256, 16, 0)                                    # token choice needs k >= 1
    assert L.moe_select(FAKE, None, None, ctypes.byref(tc0), FAKE, FAKE, None, 0, None) == \
        N.MOE_ERR_INVALID_ARG


# ---------------------------------------------------------------- GPU parity

def _run(cfg):
    from harness import compare_all, log, run_gpu
    log(f"[small] {cfg.name} n={cfg.n} d={cfg.d} E={cfg.E} k={cfg.k} dir={cfg.direction}")
    inp = W.gen_inputs(cfg)
    g = run_gpu(cfg, inp)
    return compare_all(cfg, inp, g), g, inp


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 3, 17, 64, 256])
def test_decode_token_choice_top8_swiglu(n):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cfg = W.SMALL_CONFIGS[3].scaled(f"decode_top8_n{n}", n=n, d=512, E=64, f=256)
    _run(cfg)


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 5, 33])
def test_decode_token_choice_capacity_and_groups(n):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _run(W.SMALL_CONFIGS[4].scaled(f"decode_top1_cap_n{n}", n=n))
    _run(W.SMALL_CONFIGS[5].scaled(f"decode_sigmoid_groups_n{n}", n=n))


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 3, 20])
def test_decode_expert_choice(n):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    rmap, g, inp = _run(_ec_tiny(n))
    if g["k"] == 0:
        assert g["n_kept"] == 0
        assert np.array_equal(g["out"], inp["x"])                   # bf16 residual, bit for bit
        assert g["stats"][6] == n and g["hist"][0] == n
