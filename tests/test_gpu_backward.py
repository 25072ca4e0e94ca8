"""GPU parity of the backward pass (the HIP path through the C ABI) against
the float64 backward oracle, on seeded synthetic inputs of the five reduced
workload shapes (fp32 token choice with capacity drops; expert choice; top-8
SwiGLU with a logit offset; Switch top-1 with the raw probability gate;
grouped sigmoid with a shared expert) and on crafted expert loads.

Checks, each against the oracle fed the device's own inputs of that step:
* d_gate (fp32 dot products): within 1e-4 of the row scale; dY_perm
  (gate * dOut, one rounding) within one bf16 rounding;
* dX_perm of the expert FFNs and the whole layer's dx: in every row,
  max-abs error within TOL x that row's RMS (floored at 1e-3 of the whole
  tensor's RMS).  Rows, not the whole tensor: the backward's bf16 roundings
  are relative to each row's magnitude, and row magnitudes spread widely (a
  token's dY scales with its gate; on the Zipf-skewed top-8 shape row RMS
  varies 6x inside one expert);
* the weight gradients dW1, dW2, the router's dW_g and the shared expert's:
  likewise row by row, but the row's RMS floored at 0.1 of its expert's
  gradient matrix RMS: a row of a weight gradient is a sum over the
  expert's tokens and can cancel to far below its terms (an expert with one
  or two tokens, a column of dZ whose signs balance), while each term
  carries the rounding of the stored dY, dA or dZ on the terms' scale.
  A whole expert matrix's max-abs error against its RMS would not do: the
  elements of a product of two Gaussian factors have heavy tails, and the
  rounding of the largest one alone reaches 6-7% of the matrix RMS.  fp32:
  1e-4.  bf16: 5e-2, from the arithmetic: the recomputed pre-activation A
  stays fp32, but dA = dH act'(A) (SwiGLU: d gate and d up) and H are
  stored in bf16, as bf16 autograd stores them, so every term of dX = sum_f
  dA W1 and of dW2 = dY^T H carries one rounding, <= 2^-8 relative;
  independent over the sum, they give an RMS error near 2^-8 / sqrt(3) =
  0.23% of the row's RMS, a maximum over a row's columns a few times that,
  plus the output's own rounding (up to 2^-8 of an element that can be
  several row RMS), a few per cent in all;
* dZ (fp32 on both sides from the same d_gate): within 1e-4 x RMS; the
  router's dW_g = X^T dZ from the device's dZ rounded to the layer's dtype
  (ties to even, the operand the matrix-core product takes) as the weight
  gradients above, within 1e-3: only the fp32 sums' order differs;
* the whole layer against the oracle's own chain: dx row by row as above,
  the shared expert's weight gradients (fed dOut itself) as the weight
  gradients above; dW_g, dW1 and dW2 per expert, RMS error within TOL / 5
  of that expert's matrix RMS.  In RMS, not element by element: end to end, two
  more stored roundings enter (Y in the layer's dtype feeds d_gate =
  <dOut, Y>, and dY_perm feeds dH = dY W2^T), both through sums that
  cancel, so an element of dW1 or dW_g can move by more than its own
  scale where such a sum cancelled for the few tokens behind it; the
  element-wise bar is held by the stage checks above, which feed the
  oracle the device's own intermediate values.
The routing comes from the device's logits (the oracle's forward is run on
them), as in the forward parity tests."""
import numpy as np
import pytest
import torch

from sparse_expert_dispatch_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from sparse_expert_dispatch_amd import _native
    _native.lib()


def rel_err(got, ref) -> float:
    """max-abs error / RMS over the whole tensor."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = np.sqrt((ref ** 2).mean()) if ref.size else 0.0
    err = np.abs(got - ref).max() if ref.size else 0.0
    return float(err / rms) if rms > 0 else float(err)


def grad_err(got, ref) -> float:
    """For weight gradients ([E, R, C], one matrix per expert; a 2-D matrix
    is one expert): in every row, max-abs error / that row's RMS, the RMS
    floored at 0.1 of its expert's matrix RMS (and at 1e-3 of the whole
    tensor's).  A row of dW1[e] (or of dW_g) is a sum over the expert's
    tokens and can cancel to far below its terms, while each term carries
    the rounding of the stored dY, dA or dZ on the terms' own scale; the
    floor keeps such a row from turning that rounding into a large relative
    error, and rows at their expert's scale are still held to their own."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    if ref.ndim == 2:
        ref, got = ref[None], got[None]
    whole = np.sqrt((ref ** 2).mean())
    if whole == 0:
        return float(np.abs(got).max())
    row = np.sqrt((ref ** 2).mean(axis=2))
    expert = np.sqrt((ref ** 2).reshape(ref.shape[0], -1).mean(axis=1))
    rms = np.maximum(np.maximum(row, 0.1 * expert[:, None]), 1e-3 * whole)
    return float((np.abs(got - ref).max(axis=2) / rms).max())


def fro_err(got, ref) -> float:
    """Largest over experts (the first axis; a 2-D matrix is one expert) of
    the RMS of the error / the RMS of that expert's matrix, floored at 1e-3
    of the whole tensor's RMS."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    if ref.ndim == 2:
        ref, got = ref[None], got[None]
    ref2 = ref.reshape(ref.shape[0], -1)
    err2 = got.reshape(ref.shape[0], -1) - ref2
    whole = np.sqrt((ref2 ** 2).mean())
    if whole == 0:
        return float(np.abs(got).max())
    rms = np.maximum(np.sqrt((ref2 ** 2).mean(axis=1)), 1e-3 * whole)
    return float((np.sqrt((err2 ** 2).mean(axis=1)) / rms).max())


def row_err(got, ref) -> float:
    """Largest over rows (the last axis is the row) of max-abs error / the
    row's RMS, the RMS floored at 1e-3 of the tensor's."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    ref2 = ref.reshape(-1, ref.shape[-1])
    got2 = got.reshape(-1, ref.shape[-1])
    whole = np.sqrt((ref2 ** 2).mean())
    if whole == 0:
        return float(np.abs(got2).max())
    rms = np.maximum(np.sqrt((ref2 ** 2).mean(axis=1)), 1e-3 * whole)
    return float((np.abs(got2 - ref2).max(axis=1) / rms).max())


def _run(cfg, inp=None, seed=11):
    from harness import host, log, upload, widen
    from oracle import moe_backward as B
    from oracle import moe_oracle as O
    from sparse_expert_dispatch_amd.layer import MoELayer, to_device
    log(f"[backward] {cfg.name} n={cfg.n} d={cfg.d} E={cfg.E} f={cfg.f} dir={cfg.direction}")
    inp = inp if inp is not None else W.gen_inputs(cfg)
    w = upload(cfg, inp)
    x = to_device(inp["x"])
    layer = MoELayer(cfg, w)
    layer.forward(x)
    rng = np.random.default_rng(seed)
    dout_f = rng.normal(size=(cfg.n, cfg.d)).astype(np.float32)
    dout_t = torch.from_numpy(dout_f).cuda().to(layer.out.dtype)
    g = layer.backward(x, dout_t)
    torch.cuda.synchronize()
    bf16 = cfg.dtype == "bf16"
    tol = 5e-2 if bf16 else 1e-4
    dout = host(dout_t)
    m = layer.map
    gmap = {key: host(getattr(m, key)) for key in ("expert_count", "expert_offset", "slot_token", "slot_gate",
                                                   "assign_slot", "token_offset", "token_slot")}
    n_kept = int(host(m.n_kept)[0])
    gmap["n_kept"] = n_kept
    for key in ("slot_token", "slot_gate"):
        gmap[key] = gmap[key][:n_kept]
    k = layer.k
    y_perm = host(layer.y_perm)[:n_kept]
    x_perm = host(layer.x_perm)[:n_kept]

    # combine backward on the device's Y
    dy_ref, dg_ref = B.combine_backward(dout, y_perm, gmap)
    dg = host(g["d_gate"])[:n_kept]
    scale = np.abs(dg_ref).max() if n_kept else 1.0
    assert np.abs(dg - dg_ref).max(initial=0) <= 1e-4 * scale, "d_gate"
    dy = widen(host(g["dy_perm"])[:n_kept])
    assert (np.abs(dy - dy_ref) <= (2.0 ** -8 if bf16 else 1e-6) * np.abs(dy_ref) + 1e-30).all(), "dY_perm"
    log(f"  combine backward ok ({n_kept} slots)")

    # expert FFN backward on the device's X_perm and dY
    dxp_ref, dw1_ref, dw2_ref = B.expert_ffn_backward(x_perm, gmap["expert_offset"], inp["w1"], inp["w2"],
                                                      cfg.act, host(g["dy_perm"])[:n_kept])
    e1 = row_err(widen(host(g["dx_perm"])[:n_kept]), dxp_ref)
    e2 = grad_err(host(g["dw1"]), dw1_ref)
    e3 = grad_err(host(g["dw2"]), dw2_ref)
    log(f"  FFN backward: dX_perm {e1:.3g} (x row RMS), dW1 {e2:.3g}, dW2 {e3:.3g} (x row RMS)")
    assert e1 <= tol and e2 <= tol and e3 <= tol
    counts = np.diff(gmap["expert_offset"])
    if (counts == 0).any():                                  # experts without rows: zero gradients
        assert (host(g["dw1"])[counts == 0] == 0).all() and (host(g["dw2"])[counts == 0] == 0).all()

    # gate backward from the device's d_gate and logits
    z = host(layer.logits)
    dz_ref = B.gate_backward(z, dg, gmap, cfg.direction, k, cfg.score,
                             host(layer.sel_idx) if cfg.direction == "tc" else None, cfg.norm_topk,
                             cfg.lb_coef, cfg.z_coef)
    e4 = rel_err(host(g["dz"]), dz_ref)
    # router backward on the device's operand: dZ rounded to the layer's
    # dtype (ties to even) as the matrix-core product takes it
    dz_op = host(g["dz"])
    if bf16:
        dz_op = torch.from_numpy(dz_op).to(torch.bfloat16).float().numpy()
    _, dwg_ref, _ = B.router_backward(inp["x"], inp["wg"], dz_op)
    e5 = grad_err(host(g["dwg"]), dwg_ref)
    log(f"  gate backward: dZ {e4:.3g} (x RMS); router: dW_g {e5:.3g} (x row RMS)")
    assert e4 <= 1e-4 and e5 <= 1e-3

    # whole layer against the oracle's own chain (forward on the device's logits)
    fwd = O.forward(cfg, inp, inject_logits=z)
    ref = B.layer_backward(cfg, inp, fwd, dout, z=z)
    res = {"dx": row_err(widen(host(g["dx"])), ref["dx"]), "d_offset": rel_err(host(g["d_offset"]), ref["d_offset"])}
    if cfg.shared_f:                                         # fed dOut itself: element-wise
        res["shared_dw1"] = grad_err(host(g["shared_dw1"]), ref["shared_dw1"])
        res["shared_dw2"] = grad_err(host(g["shared_dw2"]), ref["shared_dw2"])
    fro = {key: fro_err(host(g[key]), ref[key]) for key in ("dwg", "dw1", "dw2")}
    log("  layer backward: " + ", ".join(f"{key} {v:.3g}" for key, v in res.items())
        + "; weight gradients (RMS error / expert RMS): " + ", ".join(f"{key} {v:.3g}" for key, v in fro.items()))
    for key, v in res.items():
        assert v <= tol, f"{key}: {v:.3g} x RMS"
    for key, v in fro.items():
        assert v <= tol / 5, f"{key}: RMS error {v:.3g} x RMS"
    return g


@pytest.mark.parametrize("which", [1, 2, 3, 4, 5])
def test_layer_backward_matches_oracle(which):
    _run(W.SMALL_CONFIGS[which])


def test_backward_sqrtsoftplus_unnormalised_and_rank_major():
    _run(W.SMALL_CONFIGS[5].scaled("bw_sqrtsp_raw", score="sqrtsoftplus", norm_topk=False, shared_f=0))
    _run(W.SMALL_CONFIGS[4].scaled("bw_rank_major", k=2, capacity_order="rank", norm_topk=True))


def _ffn_backward_case(rows, d, f, seed):
    from harness import host, widen
    from oracle import moe_backward as B
    from sparse_expert_dispatch_amd import _native as N
    rng = np.random.default_rng(seed)
    E = len(rows)
    M = sum(rows)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    for act, fr in ((N.MOE_GELU, f), (N.MOE_SWIGLU, 2 * f)):
        def bf(a):
            return torch.from_numpy(a.astype(np.float32)).cuda().to(torch.bfloat16)
        x = bf(rng.normal(size=(M, d)))
        w1 = bf(rng.normal(size=(E, fr, d)) * d ** -0.5)
        w2 = bf(rng.normal(size=(E, d, f)) * f ** -0.5)
        dy = bf(rng.normal(size=(M, d)))
        offs = torch.from_numpy(off).cuda()
        dx = torch.empty_like(x)
        dw1 = torch.empty((E, fr, d), dtype=torch.float32, device="cuda")
        dw2 = torch.empty((E, d, f), dtype=torch.float32, device="cuda")
        ws = torch.empty(N.moe_ffn_backward_workspace_size(M, E, d, f, act, N.MOE_BF16), dtype=torch.uint8,
                         device="cuda")
        N.moe_expert_ffn_backward(x, offs, w1, w2, act, dy, dx, dw1, dw2, ws)
        torch.cuda.synchronize()
        h = [host(t) for t in (x, w1, w2, dy)]
        dx_ref, dw1_ref, dw2_ref = B.expert_ffn_backward(h[0], off, h[1], h[2], "swiglu" if act else "gelu", h[3])
        for name, err, got, ref in (("dX", row_err, widen(host(dx)), dx_ref), ("dW1", grad_err, host(dw1), dw1_ref),
                                    ("dW2", grad_err, host(dw2), dw2_ref)):
            assert err(got, ref) <= 5e-2, (act, name, err(got, ref))
        for e in range(E):
            if rows[e] == 0:
                assert (host(dw1)[e] == 0).all() and (host(dw2)[e] == 0).all()


@pytest.mark.parametrize("d,f", [(192, 64), (256, 192), (192, 128), (100, 60), (128, 102)])
def test_backward_ragged_tiles(d, f):
    """Experts of 0, 1, 31, 33, 130 and 300 rows (empty experts, K tails of
    the weight gradients, several 128-row tiles).  (192, 64): d and f not
    multiples of 128, partial column tiles everywhere, the weight gradients
    on the tiled kernel; (256, 192): dW1 (f x 256, 2f x 256) on the
    persistent weight-gradient kernel with a partial last row tile;
    (192, 128): dW2 (192 x 128) on it likewise; (100, 60): rows that are not
    whole 16-byte chunks, so every GEMM takes the plain bf16 kernel;
    (128, 102): d a multiple of 64 but f_rows not, so the recompute and dX
    stay off the forward's kernel (whose stores are whole 16-byte pieces of
    rows) and W2's 102-element rows take the plain kernel."""
    from harness import log
    log(f"[backward ragged] d={d} f={f}")
    _ffn_backward_case([0, 1, 31, 33, 130, 300], d, f, 21 + d + f)


def test_backward_wide_tiles():
    """Experts averaging more than 512 rows (0, 900, 1300, 40: empty, ragged
    last row tiles) with d = 512, f = 256: the row-grouped GEMMs whose width
    is a multiple of 256 (recompute and dH of SwiGLU, dX of both) run on the
    128 x 256 tiles."""
    from harness import log
    log("[backward wide] rows 0/900/1300/40, d=512 f=256")
    _ffn_backward_case([0, 900, 1300, 40], 512, 256, 77)


@pytest.mark.parametrize("E", [300, 512])
def test_backward_many_experts(E):
    """More experts than one wave has lanes: the weight gradients' plan deals
    them in 5 or 8 lane chunks (a fifth of the experts empty, the rest 1 to
    60 rows).  d = 256, f = 128: both weight gradients on the persistent
    kernel with the plan (output widths 256 and 128), the recompute and dX
    on the forward's LDS-tiled kernel (few rows per expert)."""
    from harness import log
    log(f"[backward many experts] E={E}")
    rng = np.random.default_rng(E)
    rows = [int(r) if rng.random() > 0.2 else 0 for r in rng.integers(1, 61, E)]
    _ffn_backward_case(rows, 256, 128, E + 5)


@pytest.mark.parametrize("i", range(16))
def test_backward_sweep_case(i):
    """The layer backward on the first 16 configurations of the forward
    sweep (tests/sweep_cases.py): every gradient against the oracle."""
    from sweep_cases import sweep_case
    _run(sweep_case(i))
