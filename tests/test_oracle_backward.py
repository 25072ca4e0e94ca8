"""Pins of the backward oracle against the forward oracle: central finite
differences of the forward functions (a gradient that drops a term, flips a
sign or transposes an operand fails them), plus the shift invariance that
softmax-based gates have.  The routing (top-k choice, capacity drops, counts)
is held fixed; the inputs keep every choice well clear of a tie, and each
check asserts the perturbed forward made the same choices.  CPU only.

Tolerances: the FFN, combine, router product and balance statistics are
float64 in the forward oracle, so their differences agree to ~1e-7; gates
and scores are specified in float32, so differences through them use a step
of 1e-3 and agree to ~1e-3 relative."""
import dataclasses

import numpy as np
import pytest

from oracle import moe_backward as B
from oracle import moe_oracle as O
from sparse_expert_dispatch_amd import workloads as W


def _fd(fun, x, v, eps):
    return (fun(x + eps * v) - fun(x - eps * v)) / (2 * eps)


def _close(a, b, rtol, scale=None):
    scale = max(abs(b), 1e-12) if scale is None else scale
    assert abs(a - b) <= rtol * scale, (a, b)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_expert_backward_finite_differences(act):
    rng = np.random.default_rng(1)
    m, d, f = 3, 5, 4
    x = rng.normal(size=(m, d))
    w1 = rng.normal(size=(2 * f if act == "swiglu" else f, d)) * 0.5
    w2 = rng.normal(size=(d, f)) * 0.5
    dy = rng.normal(size=(m, d))
    dx, dw1, dw2 = B.expert_backward(x, w1, w2, act, dy)
    L = lambda a, b, c: float((dy * O.expert_forward(a, b, c, act)).sum())
    for arg, grad in ((0, dx), (1, dw1), (2, dw2)):
        args = [x, w1, w2]
        v = rng.normal(size=args[arg].shape)

        def fun(p, arg=arg):
            a = list(args)
            a[arg] = p
            return L(*a)
        _close(_fd(fun, args[arg], v, 1e-6), float((grad * v).sum()), 1e-6)


def _tc_map(n=7, E=5, k=2, cap=3, seed=2):
    rng = np.random.default_rng(seed)
    z = (rng.permutation(n * E).reshape(n, E) * 0.11 - 2.0).astype(np.float32)   # no ties, gaps 0.11
    idx, gate = O.select_token_choice(z, k)
    rmap = O.build_map_token_choice(idx, gate, E, cap)
    return z, idx, gate, rmap


def test_combine_backward_finite_differences():
    rng = np.random.default_rng(3)
    z, idx, gate, rmap = _tc_map()
    assert (rmap["assign_slot"] < 0).any()                  # some assignments dropped
    n, d = z.shape[0], 4
    M = int(rmap["n_kept"])
    y = rng.normal(size=(M, d))
    dout = rng.normal(size=(n, d))
    dy, dg = B.combine_backward(dout, y, rmap)
    L = lambda yy, gg: float((dout * O.combine(yy, gg, rmap["token_offset"], rmap["token_slot"], n)).sum())
    v = rng.normal(size=y.shape)
    _close(_fd(lambda p: L(p, rmap["slot_gate"].astype(np.float64)), y, v, 1e-6), float((dy * v).sum()), 1e-6)
    u = rng.normal(size=M)
    _close(_fd(lambda p: L(y, p), rmap["slot_gate"].astype(np.float64), u, 1e-6), float((dg * u).sum()), 1e-6)


def test_dispatch_backward_is_the_adjoint_of_dispatch():
    rng = np.random.default_rng(4)
    z, idx, gate, rmap = _tc_map()
    n, d = z.shape[0], 3
    M = int(rmap["n_kept"])
    x = rng.normal(size=(n, d))
    g = rng.normal(size=(M, d))
    # <dispatch(x), g> == <x, dispatch_backward(g)>
    lhs = float((O.dispatch(x, rmap["slot_token"]) * g).sum())
    rhs = float((x * B.dispatch_backward(g, rmap, n)).sum())
    _close(lhs, rhs, 1e-12, scale=abs(lhs) + 1)


def _slot_gates_tc(z, idx_ref, rmap, score, norm):
    """Gates of the fixed assignments, per slot, from the forward oracle."""
    idx, gate = O.select_token_choice(z, idx_ref.shape[1], score, None, 1, 1, 1, norm)
    assert np.array_equal(idx, idx_ref), "perturbation changed the choice"
    a = rmap["assign_slot"]
    out = np.zeros(int(rmap["n_kept"]))
    out[a[a >= 0]] = gate[a >= 0]
    return out


@pytest.mark.parametrize("score,norm", [("softmax", True), ("softmax", False), ("sigmoid", True),
                                        ("sigmoid", False), ("sqrtsoftplus", True)])
def test_token_choice_gate_backward_finite_differences(score, norm):
    rng = np.random.default_rng(5)
    z, _, _, _ = _tc_map(seed=6)
    idx, gate = O.select_token_choice(z, 2, score, None, 1, 1, 1, norm)
    rmap = O.build_map_token_choice(idx, gate, z.shape[1], 3)
    M = int(rmap["n_kept"])
    dg = rng.normal(size=M)
    dz = B.gate_backward(z, dg, rmap, "tc", 2, score, idx, norm)
    assert (dz[np.ones_like(dz, bool) & ~np.isin(np.arange(z.shape[1])[None, :], idx[:, :, None]).any(1)] == 0).all()
    v = rng.normal(size=z.shape)
    L = lambda zz: float((dg * _slot_gates_tc(zz.astype(np.float32), idx, rmap, score, norm)).sum())
    _close(_fd(L, z.astype(np.float64), v, 1e-3), float((dz * v).sum()), 2e-3,
           scale=float(np.abs(dz * v).sum()))
    if score == "softmax" and norm:                          # shift invariance of a softmax
        np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-12)


def test_expert_choice_gate_backward_finite_differences():
    rng = np.random.default_rng(7)
    n, E, k = 9, 4, 3
    z = (rng.permutation(n * E).reshape(n, E) * 0.13 - 2.0).astype(np.float32)
    I, G = O.select_expert_choice(z, k)
    rmap = O.build_map_expert_choice(I, G, n)
    dg = rng.normal(size=E * k)
    dz = B.gate_backward(z, dg, rmap, "ec", k)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-12)

    def L(zz):
        I2, G2 = O.select_expert_choice(zz.astype(np.float32), k)
        assert np.array_equal(I2, I), "perturbation changed the choice"
        return float((dg * G2.reshape(-1)).sum())
    v = rng.normal(size=z.shape)
    _close(_fd(L, z.astype(np.float64), v, 1e-3), float((dz * v).sum()), 2e-3,
           scale=float(np.abs(dz * v).sum()))


@pytest.mark.parametrize("direction,score", [("tc", "softmax"), ("tc", "sigmoid"), ("tc", "sqrtsoftplus"),
                                             ("ec", "softmax")])
def test_auxiliary_loss_gradients_finite_differences(direction, score):
    rng = np.random.default_rng(8)
    n, E, k = 11, 6, 2
    z = rng.normal(size=(n, E)).astype(np.float32)
    if direction == "tc":
        idx, gate = O.select_token_choice(z, k, score)
        rmap = O.build_map_token_choice(idx, gate, E, 4)
    else:
        I, G = O.select_expert_choice(z, k)
        rmap = O.build_map_expert_choice(I, G, n)
    lb_coef, z_coef = 0.3, 0.07
    dz = B.gate_backward(z, np.zeros(int(rmap["n_kept"])), rmap, direction, k, score,
                         None if direction == "ec" else idx, True, lb_coef, z_coef)

    def L(zz):
        st, _ = O.balance_stats(zz, rmap, direction, k, score, lb_coef, z_coef)
        return st[0] + st[1]
    v = rng.normal(size=z.shape)
    _close(_fd(L, z.astype(np.float64), v, 1e-6), float((dz * v).sum()), 1e-6)


def test_router_backward_finite_differences():
    rng = np.random.default_rng(9)
    n, d, E = 5, 7, 3
    x = rng.normal(size=(n, d))
    wg = rng.normal(size=(d, E))
    dz = rng.normal(size=(n, E))
    dx, dwg, doff = B.router_backward(x, wg, dz)
    off = rng.normal(size=E).astype(np.float32)
    L = lambda a, b, o: float((dz * O.router_logits(a, b, o)).sum())
    for grad, fun, p in ((dx, lambda q: L(q, wg, off), x), (dwg, lambda q: L(x, q, off), wg),
                         (doff, lambda q: L(x, wg, q.astype(np.float32)), off.astype(np.float64))):
        v = rng.normal(size=p.shape)
        _close(_fd(fun, p, v, 1e-3), float((grad * v).sum()), 2e-3, scale=float(np.abs(grad * v).sum()) + 1e-3)


def _small_cfg(base, **kw):
    return dataclasses.replace(base, **kw)


@pytest.mark.parametrize("which", ["tc_softmax_cap_shared", "tc_sigmoid_groups", "ec_softmax"])
def test_layer_backward_finite_differences(which):
    """Whole layer: L = <dOut, out> + lb + z-loss through moe_oracle.forward,
    differentiated along random directions of x, W_g, W1 and W2."""
    if which == "tc_softmax_cap_shared":
        cfg = W.SMALL_CONFIGS[1].scaled("bw_tc", n=10, d=6, E=4, f=5, k=2, capacity_factor=0.75,
                                        shared_f=3, act="swiglu")
    elif which == "tc_sigmoid_groups":
        cfg = W.SMALL_CONFIGS[5].scaled("bw_sig", n=9, d=6, E=8, f=4, k=3, shared_f=0)
    else:
        cfg = W.SMALL_CONFIGS[2].scaled("bw_ec", n=12, d=6, E=4, f=5)
    cfg = _small_cfg(cfg, dtype="f32", lb_coef=0.2, z_coef=0.05)
    inp = W.gen_inputs(cfg)
    rng = np.random.default_rng(10)
    fl = {key: O.widen(a) if isinstance(a, np.ndarray) and a.dtype == np.uint16 else a for key, a in inp.items()}
    fl["x"] = rng.normal(size=(cfg.n, cfg.d))
    fl["wg"] = rng.normal(size=(cfg.d, cfg.E)) * 0.8
    fl["w1"] = np.asarray(fl["w1"], dtype=np.float64)
    fl["w2"] = np.asarray(fl["w2"], dtype=np.float64)
    fwd = O.forward(cfg, fl)
    dout = rng.normal(size=(cfg.n, cfg.d))
    g = B.layer_backward(cfg, fl, fwd, dout)

    def L(key, p):
        q = dict(fl)
        q[key] = p
        r = O.forward(cfg, q)
        assert np.array_equal(r["sel_idx"], fwd["sel_idx"]), "perturbation changed the choice"
        return float((dout * r["out"]).sum()) + r["stats"][0] + r["stats"][1]
    for key, grad in (("x", g["dx"]), ("wg", g["dwg"]), ("w1", g["dw1"]), ("w2", g["dw2"])):
        v = rng.normal(size=fl[key].shape)
        _close(_fd(lambda p: L(key, p), fl[key], v, 1e-4), float((grad * v).sum()), 2e-3,
               scale=float(np.abs(grad * v).sum()) + 1e-3)
