"""GPU parity of the backward pass (the HIP path through the C ABI) against
the float64 backward oracle, on seeded synthetic inputs of the five reduced
workload shapes (fp32 token choice with capacity drops; expert choice; top-8
SwiGLU with a logit offset; Switch top-1 with the raw probability gate;
grouped sigmoid with a shared expert) and on crafted expert loads.

Checks, each against the oracle fed the device's own inputs of that step:
* d_gate (fp32 dot products): within 1e-4 of the row scale; dY_perm
  (gate * dOut, one rounding) within one bf16 rounding;
* dX_perm, dW1, dW2 of the expert FFNs, the router's dX and dW_g, and the
  whole layer's dx: in every row, max-abs error within TOL x that row's RMS
  (floored at 1e-3 of the whole tensor's RMS).  Rows, not the whole tensor:
  the backward's bf16 roundings are relative to each row's magnitude, and
  row magnitudes spread widely (a token's dY scales with its gate; on the
  Zipf-skewed top-8 shape row RMS varies 6x inside one expert).  fp32:
  1e-4.  bf16: 5e-2, from the arithmetic: the recomputed pre-activation A
  stays fp32, but dA = dH act'(A) (SwiGLU: d gate and d up) and H are
  stored in bf16, as bf16 autograd stores them, so every term of dX = sum_f
  dA W1 and of dW2 = dY^T H carries one rounding, <= 2^-8 relative;
  independent over the sum, they give an RMS error near 2^-8 / sqrt(3) =
  0.23% of the row's RMS, a maximum over a row's columns a few times that,
  plus the output's own rounding (up to 2^-8 of an element that can be
  several row RMS), a few per cent in all;
* dZ (fp32 on both sides from the same d_gate): within 1e-4 x RMS.
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
    e2 = row_err(host(g["dw1"]), dw1_ref)
    e3 = row_err(host(g["dw2"]), dw2_ref)
    log(f"  FFN backward: dX_perm {e1:.3g}, dW1 {e2:.3g}, dW2 {e3:.3g} (x row RMS)")
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
    log(f"  gate backward: dZ {e4:.3g} (x RMS)")
    assert e4 <= 1e-4

    # whole layer against the oracle's own chain (forward on the device's logits)
    fwd = O.forward(cfg, inp, inject_logits=z)
    ref = B.layer_backward(cfg, inp, fwd, dout, z=z)
    res = {"dx": row_err(widen(host(g["dx"])), ref["dx"]), "dwg": row_err(host(g["dwg"]), ref["dwg"]),
           "dw1": row_err(host(g["dw1"]), ref["dw1"]), "dw2": row_err(host(g["dw2"]), ref["dw2"]),
           "d_offset": rel_err(host(g["d_offset"]), ref["d_offset"])}
    if cfg.shared_f:
        res["shared_dw1"] = row_err(host(g["shared_dw1"]), ref["shared_dw1"])
        res["shared_dw2"] = row_err(host(g["shared_dw2"]), ref["shared_dw2"])
    log("  layer backward: " + ", ".join(f"{key} {v:.3g}" for key, v in res.items()))
    for key, v in res.items():
        assert v <= tol, f"{key}: {v:.3g} x RMS"
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
        for name, got, ref in (("dX", widen(host(dx)), dx_ref), ("dW1", host(dw1), dw1_ref),
                               ("dW2", host(dw2), dw2_ref)):
            assert row_err(got, ref) <= 5e-2, (act, name, row_err(got, ref))
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
