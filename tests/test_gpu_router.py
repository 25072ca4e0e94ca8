"""The router call on its own, across the shapes its kernels tell apart.

moe_router computes Z = X W_g (+ offset, + noise_std * noise) and the
scores (page 2 "Expert choice routing", section "The math": S =
softmax(X W_g); page 5 "MoE routing strategies explained", strategy 4 for
the sigmoid scores; page 4 "How MoE routing strategies ...", section
"Pitfalls" for the noise).  For bf16 inputs with at most 64 experts one
fused kernel does it all (workgroups of 16 or 32 rows, K split over 4 or 16
waves).  65 to 128 experts: the same fused kernel with a 128-expert tile
(every softmax row whole in one workgroup).  More experts with a per-expert
score (sigmoid, sqrtsoftplus): the fused kernel on 64-expert tiles spread
over workgroups.  Softmax over more than 128 experts, or K not a multiple
of the step, takes the split-K GEMM and its finalize kernel.  Every case checks the logits against the
oracle's float64 product (within 1e-5 of each row's largest magnitude) and
the scores, row-major and transposed, bit for bit against the oracle's
score functions applied to the device's own logits."""
import numpy as np
import pytest
import torch

from sparse_expert_dispatch_amd import _native as N

pytestmark = pytest.mark.gpu

SCORES = {"softmax": N.MOE_SOFTMAX, "sigmoid": N.MOE_SIGMOID, "sqrtsoftplus": N.MOE_SQRTSOFTPLUS}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    N.lib()


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even."""
    u = a.astype(np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _run_router(n, d, E, score, with_offset=False, with_noise=False, seed=0):
    from oracle import moe_oracle as O
    from harness import check_logits, log
    log(f"[router] n={n} d={d} E={E} score={score} offset={with_offset} noise={with_noise}")
    rng = np.random.default_rng(seed)
    x = _bf16_bits(rng.normal(size=(n, d)).astype(np.float32))
    wg = _bf16_bits((rng.normal(size=(d, E)) * d ** -0.5).astype(np.float32))
    off = (rng.normal(size=E) * 0.5).astype(np.float32) if with_offset else None
    noise = rng.normal(size=(n, E)).astype(np.float32) if with_noise else None
    noise_std = 0.3 if with_noise else 0.0
    dev = "cuda"
    xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    wt = torch.from_numpy(wg.view(np.int16)).to(dev).view(torch.bfloat16)
    cfg = N.make_cfg(n, d, E, 1, N.MOE_TOKEN_CHOICE, SCORES[score])
    logits = torch.empty((n, E), dtype=torch.float32, device=dev)
    scores = torch.empty((n, E), dtype=torch.float32, device=dev)
    scores_t = torch.empty((E, n), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, N.moe_router_workspace_size(cfg, N.MOE_BF16)), dtype=torch.uint8, device=dev)
    N.moe_router(xt, wt, None if off is None else torch.from_numpy(off).to(dev), cfg, logits, scores,
                 scores_t, ws, noise=None if noise is None else torch.from_numpy(noise).to(dev),
                 noise_std=noise_std)
    torch.cuda.synchronize()
    z = logits.cpu().numpy()
    check_logits(z, O.router_logits(x, wg, off, noise, noise_std))
    s_ref = O.router_scores(z, score)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scores"
    assert np.array_equal(scores_t.cpu().numpy().view(np.uint32), s_ref.T.copy().view(np.uint32)), "scores_t"


@pytest.mark.parametrize("n,d,E,score", [
    (1, 512, 16, "softmax"),          # one row, 16-wave workgroup
    (17, 512, 32, "sigmoid"),         # ragged rows, 2 expert tiles
    (100, 1024, 48, "sqrtsoftplus"),  # 3 expert tiles (W_g columns past E never read)
    (64, 2048, 64, "softmax"),        # decode shape
    (1030, 128, 64, "softmax"),       # 65 workgroups of 4 waves, ragged last one
    (8200, 256, 64, "sigmoid"),       # 32-row workgroups, ragged last one
])
def test_fused_router_shapes(n, d, E, score):
    _run_router(n, d, E, score)


def test_fused_router_offset_and_noise():
    _run_router(300, 1024, 64, "softmax", with_offset=True, with_noise=True, seed=3)
    _run_router(4100, 256, 32, "sigmoid", with_offset=True, with_noise=True, seed=4)


@pytest.mark.parametrize("n,d,E,score", [
    (500, 512, 128, "softmax"),       # 128-expert tile, 32-row workgroups, ragged last one
    (33, 1024, 96, "sigmoid"),        # 128-expert tile with 32 columns past E
    (2100, 4096, 128, "softmax"),     # the Switch workload's router shape (d, E), fewer rows
    (700, 7168, 256, "sigmoid"),      # four 64-expert tiles: the DeepSeek-V3-shaped router (d, E)
    (129, 512, 192, "sqrtsoftplus"),  # three 64-expert tiles, ragged rows
    (4000, 256, 128, "sigmoid"),      # two 64-expert tiles, 64-row workgroups
])
def test_expert_tiled_router(n, d, E, score):
    _run_router(n, d, E, score, with_offset=True, with_noise=score == "sigmoid", seed=n)


@pytest.mark.parametrize("n,d,E,score", [
    (500, 512, 256, "softmax"),       # softmax over more than 128 experts: split-K GEMM + finalize
    (300, 96, 64, "softmax"),         # K not a multiple of 64: scalar GEMM + finalize
])
def test_other_router_paths(n, d, E, score):
    _run_router(n, d, E, score, with_offset=True)
