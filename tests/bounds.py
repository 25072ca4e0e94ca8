"""Element-wise error bounds of the bf16 device path, derived from its
rounding points, for the parity tests and the smoke check.

The device computes an expert's rows as

    A  = X W1^T               fp32 accumulation over d (matrix cores)
    h  = act(A)               fp32 (GELU with a 1.5e-7 erf, SiLU with the
                              hardware exp and reciprocal)
    hb = bf16(h)              one rounding, relative error <= u = 2^-8
    y  = hb W2^T              fp32 accumulation over f
    yb = bf16(y)              one rounding

and the combine as out = bf16(residual + shared + sum_s g_s yb_s) with fp32
accumulation (page 2 "Expert choice routing", section "The math": out =
scatter_add(G * Y, I); the residual rides beside it).  The oracle computes
the same quantities in float64 from the same bf16 inputs, without the
roundings.

Terms of the bound on |device - oracle|, per element:

* the rounding of h: sum_f delta_f h_f W2[j, f] with |delta_f| <= u.  The
  delta_f of different hidden elements are independent, zero-mean rounding
  errors (round to nearest even is unbiased), so by Hoeffding's inequality
  |sum| <= lam u sqrt(sum_f (h_f W2[j, f])^2) except with probability
  2 exp(-lam^2 / 2) -- the probabilistic rounding-error analysis of Higham
  and Mary, "A new approach to probabilistic rounding error analysis"
  (SIAM J. Sci. Comput. 41(5), 2019).  lam = 8: 2.5e-14 per element.  In the
  branch the h roundings of all the token's experts (gate-weighted) form
  one such sum.
* the fp32 accumulations over d and f: lam sqrt(K) 2^-24 sum |a_i b_i| (the
  same analysis at fp32's unit roundoff), the d-sum's error carried to h by
  |act'| <= 1.2 and on through |W2|.
* the activation functions' own error: 1e-6 relative of h (and of A for
  GELU), far above their 1.5e-7 / few-ulp error.
* the roundings of y and of the output: u |y| per expert row (gate-weighted
  in the branch) and u |out|, deterministic.
* the combine's fp32 sum of at most k + 2 terms: (k + 2) 2^-24 sum |terms|.

No term is a tolerance chosen to pass: each is the size of one rounding
point of the device's arithmetic.  fp32 layers keep a plain 1e-4 x RMS
check (no bf16 rounding anywhere).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import moe_oracle as O

U_BF16 = 2.0 ** -8          # unit roundoff of bf16, round to nearest even
U_F32 = 2.0 ** -24          # unit roundoff of fp32
LAM = 8.0                   # probabilistic bound constant (Hoeffding / Higham-Mary)
ACT_LIP = 1.2               # |gelu'| <= 1.13, |silu'| <= 1.1
ACT_REL = 1e-6              # activation-function error, relative


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


class ExpertRows:
    """One expert's oracle rows and the pieces of their device-error bound.

    y      oracle output rows (float64, O.expert_forward)
    s2     sum_f (h_f W2[j, f])^2: the variance scale of the h rounding
    det    deterministic fp32-level terms (accumulations, activation error)
    """

    def __init__(self, xe: np.ndarray, w1: np.ndarray, w2: np.ndarray, act: str):
        x = widen(xe)
        W1 = widen(w1)
        W2 = widen(w2)
        d = x.shape[1]
        f = W2.shape[1]
        h = O.expert_hidden(xe, w1, act)             # the oracle's hidden activation
        self.y = h @ W2.T
        A = x @ W1.T                                  # pre-activation magnitudes, for the bound only
        SA = np.abs(x) @ np.abs(W1).T                 # sum_k |x_k w_k| per pre-activation
        c_d = LAM * math.sqrt(d) * U_F32
        if act == "gelu":
            eh = ACT_LIP * c_d * SA + ACT_REL * (np.abs(h) + np.abs(A))
        else:
            g, up = A[:, :f], A[:, f:]
            sg = O.silu(g)
            eh = c_d * (ACT_LIP * np.abs(up) * SA[:, :f] + np.abs(sg) * SA[:, f:]) + ACT_REL * np.abs(h)
        aW2 = np.abs(W2)
        ah = np.abs(h)
        self.s2 = (h * h) @ (W2 * W2).T
        self.det = eh @ aW2.T + LAM * math.sqrt(f) * U_F32 * (ah @ aW2.T)

    def bound(self) -> np.ndarray:
        """|yb - y| <= (1 + u) (lam u sqrt(s2) + det) + u |y|."""
        return (1 + U_BF16) * (LAM * U_BF16 * np.sqrt(self.s2) + self.det) + U_BF16 * np.abs(self.y)


def check_rows(y_dev: np.ndarray, rows: ExpertRows, what: str) -> float:
    """Device bf16 expert rows within their bound; returns max-abs / RMS(y)."""
    got = widen(y_dev)
    excess = np.abs(got - rows.y) - rows.bound()
    rms = float(np.sqrt((rows.y ** 2).mean()))
    err = float(np.abs(got - rows.y).max() / rms) if rms > 0 else 0.0
    assert excess.max() <= 0, f"{what}: error exceeds the rounding bound by {excess.max():.3g} " \
                              f"(max-abs / RMS {err:.3g})"
    return err


class BranchBound:
    """Accumulates, token by token, the oracle branch and its bound:
    sum over the token's kept slots of g_s y_s (plus the shared expert with
    weight 1).  `add(i, g, rows, r)` adds row r of an ExpertRows with gate g
    to token i."""

    def __init__(self, n_tok: int, d: int):
        self.branch = np.zeros((n_tok, d))
        self.lin = np.zeros((n_tok, d))       # sum |g| (u |y| + det)
        self.var = np.zeros((n_tok, d))       # sum g^2 s2
        self.mag = np.zeros((n_tok, d))       # sum |g y|: the combine's fp32 terms
        self.terms = np.zeros(n_tok, dtype=np.int64)

    def add(self, i: int, g: float, rows: ExpertRows, r: int):
        y = rows.y[r]
        self.branch[i] += g * y
        self.lin[i] += abs(g) * (U_BF16 * np.abs(y) + rows.det[r])
        self.var[i] += g * g * rows.s2[r]
        self.mag[i] += np.abs(g * y)
        self.terms[i] += 1

    def bound(self, residual: np.ndarray = None) -> np.ndarray:
        """Bound on |device - oracle| for the branch (residual None) or for
        residual + branch."""
        rest = (1 + U_BF16) * (self.lin + LAM * U_BF16 * np.sqrt(self.var))
        total = self.branch if residual is None else self.branch + residual
        mag = self.mag if residual is None else self.mag + np.abs(residual)
        acc = (self.terms[:, None] + 2) * U_F32 * mag
        return rest + acc + U_BF16 * (np.abs(total) + rest + acc)


def check_branch(got: np.ndarray, bb: BranchBound, residual: np.ndarray = None, what: str = "branch"):
    """Device branch (or residual + branch) within the composed bound.
    Returns (max-abs / RMS, the same for one bf16 rounding of the exact
    result alone, the largest bound / RMS)."""
    ref = bb.branch if residual is None else bb.branch + residual
    g = widen(got)
    bound = bb.bound(residual)
    excess = np.abs(g - ref) - bound
    rms = float(np.sqrt((ref ** 2).mean()))
    err = float(np.abs(g - ref).max() / rms)
    r32 = ref.astype(np.float32)
    u = r32.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    floor = float(np.abs(rounded.view(np.float32).astype(np.float64) - ref).max() / rms)
    assert excess.max() <= 0, f"{what}: error exceeds the derived bound by {excess.max():.3g} " \
                              f"at {np.unravel_index(np.argmax(excess), excess.shape)} " \
                              f"(max-abs / RMS {err:.3g})"
    return err, floor, float(bound.max() / rms)


def _kept_slots(rmap: dict, t: int) -> list:
    a, b = int(rmap["token_offset"][t]), int(rmap["token_offset"][t + 1])
    return [int(s) for s in rmap["token_slot"][a:b] if s >= 0]


def check_layer_rows(cfg, inp: dict, rmap: dict, tokens, y_perm_dev: np.ndarray, shared_dev=None,
                     progress=None):
    """Every expert row that `tokens` use (and their shared-expert rows)
    within its rounding bound, one expert at a time; returns the
    BranchBound of those tokens and the worst row max-abs / RMS(y)."""
    tokens = np.asarray(tokens)
    bb = BranchBound(len(tokens), cfg.d)
    pairs = {}                                       # expert -> [(token position, slot)]
    for i, t in enumerate(tokens):
        for s in _kept_slots(rmap, t):
            e = int(np.searchsorted(rmap["expert_offset"], s, side="right") - 1)
            pairs.setdefault(e, []).append((i, s))
    worst = 0.0
    for done, (e, lst) in enumerate(sorted(pairs.items())):
        if progress is not None and done % 32 == 31:
            progress(f"  expert rows: {done + 1} of {len(pairs)} experts checked")
        slots = [s for _, s in lst]
        R = ExpertRows(inp["x"][rmap["slot_token"][slots]], inp["w1"][e], inp["w2"][e], cfg.act)
        worst = max(worst, check_rows(y_perm_dev[slots], R, f"expert {e}"))
        for r, (i, s) in enumerate(lst):
            bb.add(i, float(rmap["slot_gate"][s]), R, r)
    if getattr(cfg, "shared_f", 0):
        R = ExpertRows(inp["x"][tokens], inp["shared_w1"], inp["shared_w2"], cfg.act)
        worst = max(worst, check_rows(shared_dev[tokens], R, "shared expert"))
        for i in range(len(tokens)):
            bb.add(i, 1.0, R, i)
    return bb, worst
