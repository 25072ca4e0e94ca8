"""CPU oracle for the MoE-layer backward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path never calls it and it never imports
the product.  It differentiates the forward that ``moe_oracle`` defines, in
float64, with the routing decisions held fixed (the top-k choice, the
capacity drops and the per-expert counts are piecewise constant in the
logits, so their derivative is zero almost everywhere).

The objective whose gradient is taken is

    L = <dOut, out> + lb_loss + z_loss,

where dOut is the gradient arriving from above, out is the layer output
(residual + shared expert + sum over kept assignments of gate * Y), and the
two auxiliary losses are the ones ``balance_stats`` reports, already scaled
by their coefficients.  The pages describe the forward only; this reading
(the auxiliary losses enter the training objective added to the task loss,
with the coefficients of page 1 "What each direction guarantees") is what
those coefficients are for.

Step by step (every product and sum in float64):

* combine   out_t = res_t + shared_t + sum_s g_s Y_s    ->  dY_s = g_s dOut_t,
            dg_s = <dOut_t, Y_s>, d res = d shared = dOut
* experts   H = act(X W1^T) (SwiGLU: silu(X Wg^T) * (X Wu^T)), Y = H W2^T
            ->  dH = dY W2, dA = dH * act'(pre-activation), dX = dA W1,
            dW2 = dY^T H, dW1 = dA^T X  (per expert, over its rows)
* dispatch  X_perm[s] = X[token(s)]  ->  dX_t = sum over t's kept slots of dX_perm[s]
* gates     token choice: softmax over the k selected logits, the full-row
            softmax probability, or a per-expert score (sigmoid,
            sqrtsoftplus) renormalised over the k or raw; expert choice: the
            row softmax S[t, e].  A dropped assignment's gate reaches no
            output, so its dg is zero (it still takes part in the
            renormalisation of the kept ones).
* losses    lb = coef E sum_e f_e P_e with f_e constant and P_e = mean_t p_te
            (p the softmax, or the score over its row sum); z = coef
            mean_t lse_t^2  ->  d lse_t / d z_te = softmax(z_t)_e.
* router    z = X W_g (+ offset, + noise_std noise)  ->  dX += dz W_g^T,
            dW_g = X^T dz, d offset = sum_t dz_t.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import moe_oracle as O


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    return O.widen(a) if a.dtype == np.uint16 else a.astype(np.float64)


# ---------------------------------------------------------------------------
# Activations and their derivatives (float64)
# ---------------------------------------------------------------------------


def gelu_grad(h: np.ndarray) -> np.ndarray:
    """d/dh of h Phi(h): Phi(h) + h phi(h)."""
    from scipy.special import erf
    phi = np.exp(-0.5 * h * h) / math.sqrt(2.0 * math.pi)
    return 0.5 * (1.0 + erf(h / math.sqrt(2.0))) + h * phi


def sigmoid64(h: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-h))


def silu_grad(h: np.ndarray) -> np.ndarray:
    """d/dh of h sigmoid(h): sigmoid(h) (1 + h (1 - sigmoid(h)))."""
    s = sigmoid64(h)
    return s * (1.0 + h * (1.0 - s))


# ---------------------------------------------------------------------------
# Expert FFN
# ---------------------------------------------------------------------------


def expert_backward(xe, w1, w2, act: str, dy):
    """One expert: Y = H W2^T with H the hidden activation of moe_oracle.
    Returns dX [m, d], dW1 [f_rows, d], dW2 [d, f] in float64."""
    x = _f64(xe)
    W1 = _f64(w1)
    W2 = _f64(w2)
    g = _f64(dy)
    pre = x @ W1.T                                   # [m, f_rows]
    if act == "gelu":
        h = O.gelu(pre)
        dh = g @ W2                                  # [m, f]
        da = dh * gelu_grad(pre)
    else:
        f = W1.shape[0] // 2
        gp, up = pre[:, :f], pre[:, f:]
        h = O.silu(gp) * up
        dh = g @ W2
        da = np.concatenate([dh * up * silu_grad(gp), dh * O.silu(gp)], axis=1)
    dx = da @ W1
    dW1 = da.T @ x
    dW2 = g.T @ h
    return dx, dW1, dW2


def expert_ffn_backward(x_perm, expert_offset, w1, w2, act: str, dy_perm):
    """Grouped over the expert-major buffer: rows offset[e]..offset[e+1] of
    X_perm and dY_perm belong to expert e.  Experts without rows get zero
    weight gradients."""
    off = np.asarray(expert_offset, dtype=np.int64)
    E = len(off) - 1
    M = int(off[-1])
    d = np.asarray(x_perm).shape[1]
    dx = np.zeros((M, d))
    dW1 = np.zeros(np.asarray(w1).shape)
    dW2 = np.zeros(np.asarray(w2).shape)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            dx[a:b], dW1[e], dW2[e] = expert_backward(np.asarray(x_perm)[a:b], w1[e], w2[e], act,
                                                      np.asarray(dy_perm)[a:b])
    return dx, dW1, dW2


# ---------------------------------------------------------------------------
# Combine and dispatch
# ---------------------------------------------------------------------------


def combine_backward(dout, y_perm, rmap: dict):
    """For every kept slot s of token t: dY_s = g_s dOut_t and dg_s =
    <dOut_t, Y_s>.  Returns dY_perm [M, d] and d_gate [M] (float64)."""
    g = _f64(dout)
    y = _f64(y_perm)
    st = np.asarray(rmap["slot_token"], dtype=np.int64)
    gate = np.asarray(rmap["slot_gate"], dtype=np.float64)
    dy = gate[:, None] * g[st]
    dgate = (g[st] * y).sum(axis=1)
    return dy, dgate


def dispatch_backward(dx_perm, rmap: dict, n: int, base=None):
    """dX_t = base_t + the sum of dX_perm over token t's kept slots."""
    dxp = _f64(dx_perm)
    out = np.zeros((n, dxp.shape[1])) if base is None else _f64(base).copy()
    to = np.asarray(rmap["token_offset"], dtype=np.int64)
    ts = np.asarray(rmap["token_slot"], dtype=np.int64)
    for t in range(n):
        for q in range(to[t], to[t + 1]):
            if ts[q] >= 0:
                out[t] += dxp[ts[q]]
    return out


# ---------------------------------------------------------------------------
# Gates and auxiliary losses -> logits
# ---------------------------------------------------------------------------


def _score64(z, score: str):
    """Per-expert score and its derivative, float64."""
    if score == "sigmoid":
        s = sigmoid64(z)
        return s, s * (1.0 - s)
    sp = np.logaddexp(0.0, z)
    r = np.sqrt(sp)
    return r, sigmoid64(z) / (2.0 * r)


def _softmax64(z):
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def gate_backward(z, d_gate, rmap: dict, direction: str, k: int, score: str = "softmax",
                  sel_idx=None, norm_topk: bool = True, lb_coef: float = 0.0, z_coef: float = 0.0):
    """d(gate part + lb + z-loss)/dz for logits z [n, E] (float32 values,
    differentiated in float64).  d_gate [M] is per slot (zero for slots that
    do not exist); token choice reads assignment (t, j)'s slot from
    assign_slot [n, k] (-1: dropped, dg = 0) and its expert from sel_idx;
    expert choice slot e*k + j is (slot_token, e)."""
    z = np.asarray(z, dtype=np.float64)
    n, E = z.shape
    dz = np.zeros((n, E))
    dg_slot = np.asarray(d_gate, dtype=np.float64)
    if direction == "tc":
        idx = np.asarray(sel_idx, dtype=np.int64)
        aslot = np.asarray(rmap["assign_slot"], dtype=np.int64).reshape(n, k)
        dg = np.where(aslot >= 0, dg_slot[np.maximum(aslot, 0)] if dg_slot.size else 0.0, 0.0)
        rows = np.arange(n)[:, None]
        zs = z[rows, idx]                                   # [n, k] selected logits
        if score == "softmax":
            if norm_topk:                                   # softmax over the selected logits
                g = _softmax64(zs)
                dzs = g * (dg - (g * dg).sum(axis=1, keepdims=True))
                np.add.at(dz, (np.repeat(np.arange(n), k), idx.reshape(-1)), dzs.reshape(-1))
            else:                                           # full-row softmax probability
                p = _softmax64(z)
                dp = np.zeros((n, E))
                np.add.at(dp, (np.repeat(np.arange(n), k), idx.reshape(-1)), dg.reshape(-1))
                dz += p * (dp - (p * dp).sum(axis=1, keepdims=True))
        else:
            r, rp = _score64(zs, score)
            if norm_topk:                                   # r_j / sum of the k
                R = r.sum(axis=1, keepdims=True)
                g = r / R
                dr = (dg - (g * dg).sum(axis=1, keepdims=True)) / R
            else:
                dr = dg
            np.add.at(dz, (np.repeat(np.arange(n), k), idx.reshape(-1)), (dr * rp).reshape(-1))
    else:
        S = _softmax64(z)
        st = np.asarray(rmap["slot_token"], dtype=np.int64)
        M = st.shape[0]
        e_of = np.arange(M) // max(k, 1)
        dS = np.zeros((n, E))
        if M:
            np.add.at(dS, (st, e_of), dg_slot[:M])
        dz += S * (dS - (S * dS).sum(axis=1, keepdims=True))
    # load-balance loss: c_e = coef E f_e / n on every p_te
    count = np.asarray(rmap["expert_count"], dtype=np.float64)
    if lb_coef and count.sum() > 0:
        c = lb_coef * E * (count / count.sum()) / n
        if score == "softmax":
            p = _softmax64(z)
            dz += p * (c[None, :] - (p * c[None, :]).sum(axis=1, keepdims=True))
        else:
            r, rp = _score64(z, score)
            R = r.sum(axis=1, keepdims=True)
            p = r / R
            dz += rp * (c[None, :] - (p * c[None, :]).sum(axis=1, keepdims=True)) / R
    # z-loss: coef mean_t lse_t^2
    if z_coef:
        m = z.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
        dz += z_coef * (2.0 / n) * lse[:, None] * _softmax64(z)
    return dz


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------


def router_backward(x, wg, dz, base=None):
    """z = X W_g (+ offset + noise): dX = base + dz W_g^T [n, d], dW_g =
    X^T dz [d, E], d offset = column sums of dz [E]."""
    X = _f64(x)
    W = _f64(wg)
    g = np.asarray(dz, dtype=np.float64)
    dx = g @ W.T
    if base is not None:
        dx = dx + _f64(base)
    return dx, X.T @ g, g.sum(axis=0)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------


def layer_backward(cfg, inp: dict, fwd: dict, dout, z: Optional[np.ndarray] = None):
    """Gradients of L = <dOut, out> + lb + z-loss for one forward `fwd` (the
    dict moe_oracle.forward returns; its map and selection are the fixed
    routing).  `z` overrides the logits the gates and losses are
    differentiated at (a device's own float32 logits).  Returns dx, dwg,
    d_offset, dw1, dw2 (and shared_dw1, shared_dw2 with a shared expert),
    plus the intermediates dy_perm, d_gate, dx_perm, dz."""
    rmap = fwd["map"]
    n = cfg.n
    z = fwd["logits"] if z is None else z
    k = fwd["k"]
    x = inp["x"]
    dy_perm, d_gate = combine_backward(dout, fwd["y_perm"], rmap)
    dx_perm, dw1, dw2 = expert_ffn_backward(fwd["x_perm"], rmap["expert_offset"], inp["w1"], inp["w2"],
                                            cfg.act, dy_perm)
    dz = gate_backward(z, d_gate, rmap, cfg.direction, k, cfg.score, fwd.get("sel_idx"),
                       cfg.norm_topk, cfg.lb_coef, cfg.z_coef)
    res = dict(dy_perm=dy_perm, d_gate=d_gate, dx_perm=dx_perm, dz=dz, dw1=dw1, dw2=dw2)
    base = _f64(dout)                                # the residual path
    if cfg.shared_f:
        dxs, res["shared_dw1"], res["shared_dw2"] = expert_backward(x, inp["shared_w1"], inp["shared_w2"],
                                                                    cfg.act, dout)
        base = base + dxs
    dx_r, res["dwg"], res["d_offset"] = router_backward(x, inp["wg"], dz, base)
    res["dx"] = dispatch_backward(dx_perm, rmap, n, dx_r)
    return res
