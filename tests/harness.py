"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
(via the Python binding), bring every stage's result back, and compare it
with the CPU oracle run on the same seeded inputs.

Selection, routing maps, drop sets and permutations must match bit for bit
given the device's fp32 logits (the oracle is run with those logits
injected).  Logits must match within 1e-5 relative to each row's largest
magnitude.  bf16 expert outputs, the MoE branch (residual = NULL) and
residual + branch must each lie, element by element, within the bound
derived from the device's rounding points (tests/bounds.py); fp32 layers
within 1e-4 x RMS of the branch."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

from oracle import moe_oracle as O
from sparse_expert_dispatch_amd import _native as N
from sparse_expert_dispatch_amd.layer import MoELayer, to_device

from bounds import check_branch, check_layer_rows

LOGIT_RTOL = 1e-5
F32_TOL = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def upload(cfg, inp: dict) -> dict:
    w = {"wg": to_device(inp["wg"]), "w1": to_device(inp["w1"]), "w2": to_device(inp["w2"]),
         "logit_offset": to_device(inp.get("logit_offset")), "sel_bias": to_device(inp.get("sel_bias")),
         "noise": to_device(inp.get("noise"))}
    if cfg.shared_f:
        w["shared_w1"] = to_device(inp["shared_w1"])
        w["shared_w2"] = to_device(inp["shared_w2"])
    return w


def run_gpu(cfg, inp: dict, weights=None) -> dict:
    """Run every stage on the GPU; return host copies of all results."""
    w = weights if weights is not None else upload(cfg, inp)
    x = to_device(inp["x"])
    layer = MoELayer(cfg, w)
    layer.route(x)
    layer.experts(x)
    layer.dispatch(x)            # the standalone gather too (the packed FFN fuses it)
    layer.combine(x, residual=False)
    branch = layer.out.clone()
    layer.combine(x, residual=True)
    layer.balance_stats()
    torch.cuda.synchronize()
    m = layer.map
    r = dict(logits=host(layer.logits), sel_idx=host(layer.sel_idx), sel_gate=host(layer.sel_gate),
             n_kept=int(host(m.n_kept)[0]), M_max=layer.M_max, k=layer.k, capacity=layer.capacity,
             expert_count=host(m.expert_count), expert_offset=host(m.expert_offset),
             slot_token=host(m.slot_token), slot_gate=host(m.slot_gate),
             assign_slot=host(m.assign_slot), token_offset=host(m.token_offset),
             token_slot=host(m.token_slot), x_perm=host(layer.x_perm), y_perm=host(layer.y_perm),
             branch=host(branch), out=host(layer.out), stats=host(layer.stats), hist=host(layer.hist))
    if layer.scores_t is not None:
        r["scores_t"] = host(layer.scores_t)
    if layer.shared:
        r["shared"] = host(layer.shared_out)
    r["layer"] = layer
    return r


def kept_slots(rmap: dict, t: int) -> list:
    """Token t's kept slots, in its list order (negative entries are drops)."""
    a, b = int(rmap["token_offset"][t]), int(rmap["token_offset"][t + 1])
    return [int(s) for s in rmap["token_slot"][a:b] if s >= 0]


def check_logits(z_gpu: np.ndarray, z_ref: np.ndarray):
    err = np.abs(z_gpu.astype(np.float64) - z_ref.astype(np.float64)).max(axis=1)
    scale = np.abs(z_ref.astype(np.float64)).max(axis=1)
    bad = err > LOGIT_RTOL * scale
    assert not bad.any(), f"logit rows off: {np.where(bad)[0][:5]}, worst rel " \
                          f"{(err / np.maximum(scale, 1e-30)).max():.3g}"


def max_rel_rms(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt((ref ** 2).mean())
    return float(np.abs(got - ref).max() / rms) if rms > 0 else float(np.abs(got - ref).max())


def check_map(g: dict, ref_map: dict):
    nk = int(ref_map["n_kept"])
    assert g["n_kept"] == nk
    for key in ("expert_count", "expert_offset", "assign_slot", "token_offset"):
        assert np.array_equal(g[key], ref_map[key]), key
    for key in ("slot_token", "slot_gate", "token_slot"):
        ln = nk if key != "token_slot" else int(ref_map["token_offset"][-1])
        got = g[key][:ln]
        want = ref_map[key][:ln]
        if key == "slot_gate":
            assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32)), key
        else:
            assert np.array_equal(got, want), key


def compare_all(cfg, inp: dict, g: dict, full_ffn: bool = True, sample_tokens=None):
    """Stage-by-stage comparison of a GPU run `g` with the oracle."""
    t0 = time.time()
    z_ref = O.router_logits(inp["x"], inp["wg"], inp.get("logit_offset"), inp.get("noise"),
                            getattr(cfg, "noise_std", 0.0))
    check_logits(g["logits"], z_ref)
    z = g["logits"]
    bf16 = cfg.dtype == "bf16"

    if cfg.direction == "tc":
        idx, gate = O.select_token_choice(z, cfg.k, cfg.score, inp.get("sel_bias"), cfg.n_group,
                                          cfg.topk_group, cfg.group_topm, cfg.norm_topk)
        cap = O.tc_capacity(cfg.n, cfg.k, cfg.E, cfg.capacity_factor)
        assert g["capacity"] == (cap if cfg.capacity_factor is not None else -1)
        rmap = O.build_map_token_choice(idx, gate, cfg.E, None if cfg.capacity_factor is None else cap,
                                        getattr(cfg, "capacity_order", "token"))
        k = cfg.k
    else:
        k = O.ec_k(cfg.n, cfg.c, cfg.E)
        assert g["k"] == k
        S = O.softmax_rows(z)
        assert np.array_equal(g["scores_t"].view(np.uint32), S.T.copy().view(np.uint32)), "scores_t"
        idx, gate = O.select_expert_choice(z, k)
        rmap = O.build_map_expert_choice(idx, gate, cfg.n)
    assert np.array_equal(g["sel_idx"], idx), "selection"
    assert np.array_equal(g["sel_gate"].view(np.uint32), gate.view(np.uint32)), "gates"
    check_map(g, rmap)
    nk = rmap["n_kept"]
    assert np.array_equal(g["x_perm"][:nk], inp["x"][rmap["slot_token"]]), "dispatch"
    log(f"  routing exact ({time.time() - t0:.1f}s)")

    w1_of = lambda e: inp["w1"][e]
    w2_of = lambda e: inp["w2"][e]
    if full_ffn:
        tokens = np.arange(cfg.n)
    else:
        tokens = np.asarray(sample_tokens)
    nt = len(tokens)
    if bf16:
        # every expert output within the bound of its rounding points, and the
        # branch (residual = NULL) within the bound composed from those
        # through the gates and the combine's rounding (tests/bounds.py)
        bb, worst = check_layer_rows(cfg, inp, rmap, tokens, g["y_perm"], g.get("shared"), progress=log)
        if full_ffn:
            # the composed branch is the oracle's: its grouped FFN and combine
            y_ref = O.expert_ffn(inp["x"][rmap["slot_token"]], rmap["expert_offset"], w1_of, w2_of, cfg.act)
            shared = (O.expert_forward(inp["x"], inp["shared_w1"], inp["shared_w2"], cfg.act)
                      if cfg.shared_f else None)
            branch = O.combine(y_ref, rmap["slot_gate"], rmap["token_offset"], rmap["token_slot"], cfg.n,
                               None, shared)
            assert np.allclose(bb.branch, branch, rtol=1e-9, atol=1e-12 * np.abs(branch).max()), "oracle branch"
        log(f"  expert rows within their rounding bound (worst max-abs / RMS {worst:.3g})")
    else:
        y_ref = O.expert_ffn(inp["x"][rmap["slot_token"]], rmap["expert_offset"], w1_of, w2_of, cfg.act)
        off = rmap["expert_offset"]
        for e in range(cfg.E):
            a, b = int(off[e]), int(off[e + 1])
            if b > a:
                err = max_rel_rms(widen(g["y_perm"][a:b]), y_ref[a:b])
                assert err <= F32_TOL, f"expert {e}: max-abs / RMS = {err:.3g}"
        shared = O.expert_forward(inp["x"], inp["shared_w1"], inp["shared_w2"], cfg.act) if cfg.shared_f else None
        branch = O.combine(y_ref, rmap["slot_gate"], rmap["token_offset"], rmap["token_slot"], cfg.n,
                           None, shared)[tokens]
    # combine on its own: the device's expert outputs summed by the oracle;
    # the only difference left is one rounding of the fp32 sum to `dtype`
    gb = widen(g["branch"][tokens])
    y_dev = widen(g["y_perm"][:rmap["n_kept"]])          # rows past n_kept are never written
    sh_dev = widen(g["shared"]) if cfg.shared_f else None
    comb = np.zeros((len(tokens), cfg.d))
    for i, t in enumerate(tokens):
        for s in kept_slots(rmap, t):
            comb[i] += float(rmap["slot_gate"][s]) * y_dev[s]
        if sh_dev is not None:
            comb[i] += sh_dev[t]
    ulp = 2.0 ** -8 if bf16 else 2.0 ** -22
    cerr = np.abs(gb - comb) - ulp * np.abs(comb)
    assert cerr.max() <= 1e-6 * np.sqrt((comb ** 2).mean()) + 1e-30, \
        f"combine: worst excess {cerr.max():.3g}"
    # the layer against the oracle end to end: the MoE branch alone
    # (residual = NULL), then residual + branch
    res = widen(inp["x"][tokens])
    if bf16:
        err_b, floor_b, bnd_b = check_branch(g["branch"][tokens], bb, None, "layer branch")
        err_o, _, _ = check_branch(g["out"][tokens], bb, res, "layer output")
        log(f"  branch: max-abs / RMS(branch) {err_b:.3g} (one bf16 rounding of the exact branch alone: "
            f"{floor_b:.3g}; largest bound / RMS {bnd_b:.3g}); residual + branch: max-abs / RMS(out) {err_o:.3g}")
    else:
        err_b = max_rel_rms(gb, branch)
        err_o = max_rel_rms(widen(g["out"][tokens]), branch + res)
        log(f"  branch: max-abs / RMS(branch) {err_b:.3g}; residual + branch: max-abs / RMS(out) {err_o:.3g}")
        assert err_b <= F32_TOL, f"layer branch: max-abs / RMS(branch) = {err_b:.3g}"
        assert err_o <= F32_TOL, f"layer output: max-abs / RMS(out) = {err_o:.3g}"
    # tokens with no kept expert (and no shared expert) ride the residual bit for bit
    if not cfg.shared_f:
        empty = np.array([t for t in tokens if not kept_slots(rmap, t)], dtype=np.int64)
        assert np.array_equal(g["out"][empty], inp["x"][empty]), "residual pass-through"
    log(f"  outputs within tolerance ({time.time() - t0:.1f}s)")

    st_ref, hist_ref = O.balance_stats(z, rmap, cfg.direction, k, cfg.score, cfg.lb_coef, cfg.z_coef)
    st = g["stats"].astype(np.float64)
    for i in range(4):
        assert abs(st[i] - st_ref[i]) <= 1e-4 * max(abs(st_ref[i]), 1e-6), \
            f"{O.STAT_NAMES[i]}: {st[i]} vs {st_ref[i]}"
    assert np.array_equal(st[4:], st_ref[4:]), (st[4:], st_ref[4:])
    assert np.array_equal(g["hist"], hist_ref)
    return rmap
