"""CPU oracle for the MoE-layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python
binding) never calls it, and this module never imports the product: the two
share no code.  Inputs arrive as plain numpy arrays (float32, or bfloat16 as
uint16 bit patterns).

It is the plain definition of what the layer computes, written out slowly:

* router     S = softmax(X W_g) (or a sigmoid per expert)      -- page 2 "The math",
                                                                  page 5 strategy 4
* selection  token choice: the k best experts of each token (a row)
             (page 2 "Token-choice and its load-balance headache"; page 5
             strategies 1, 2, 4, 5); expert choice: the k best tokens of each expert
             of each column, k = n c / E (page 1 "Who picks whom"; page 2
             "The transposed selection", "The math")
* routing    capacity per expert, tokens arriving after the buffer is full skip
             the expert and ride the residual (page 1 "Dropped tokens flow in
             opposite directions"; page 5 strategy 2); dropless keeps all
* dispatch   X_in[e] = P[e] X with P the one-hot of the chosen indices
* experts    per-expert FFN (GELU or SwiGLU)
* combine    out = scatter_add(gate * Y, I), plus the residual and the
             always-on shared expert (page 2 "The math"; page 5 strategy 3)
* statistics load-balance loss, router z-loss (page 1 "What each direction
             guarantees"), MaxVio (page 5 TL;DR)

Floating point is float64 unless a step is *specified* in float32 so that
the GPU can reproduce it bit for bit given the same float32 logits: the
score transform (``spec_exp``, the softmax tree sum, the sigmoid) and the
gates.  Those steps are written as single float32 operations in a fixed
order, with no fused multiply-add.

Where the pages leave a step open, the reading taken is stated at the
function.  ``balance_stats``' load-balance loss, z-loss and MaxVio formulas
are readings (the pages give names and coefficients only); they are pinned by
closed forms, not by printed values.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

f32 = np.float32

# ---------------------------------------------------------------------------
# Input widening
# ---------------------------------------------------------------------------


def widen(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) or float32 -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# Specified float32 exp (Cody & Waite argument reduction, Taylor polynomial)
# ---------------------------------------------------------------------------
# x = k ln2 + r with k = nearest integer to x/ln2 and |r| <~ ln2/2, so
# e^x = 2^k e^r.  ln2 is split into a high part with 9 zero low-order
# mantissa bits (so k*LN2_HI is exact for |k| < 2^9) and the float32 rounding
# of the remainder.  e^r is the degree-7 Taylor polynomial in Horner form;
# its truncation error at |r| = ln2/2 is below 6e-9 relative.
LOG2E = f32(1.0 / math.log(2.0))
LN2_HI = (np.array([math.log(2.0)], dtype=np.float32).view(np.uint32)
          & np.uint32(0xFFFFFE00)).view(np.float32)[0]
LN2_LO = f32(math.log(2.0) - float(LN2_HI))
INV_FACT = [f32(1.0 / math.factorial(j)) for j in range(8)]   # 1/j!, j = 0..7
EXP_LO = f32(-86.0)   # below: 0 (keeps every non-zero result a normal float)
EXP_HI = f32(88.0)    # above: +inf


def spec_exp(x) -> np.ndarray:
    """Specified float32 exp; every step one IEEE float32 operation."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        kf = np.rint(x * LOG2E)                      # float32 multiply, round half even
        r = (x - kf * LN2_HI) - kf * LN2_LO          # k*LN2_HI exact; two roundings after
        p = INV_FACT[7]
        for j in range(6, -1, -1):                   # Horner: p = p*r + 1/j!
            p = p * r + INV_FACT[j]
        p = np.asarray(p, dtype=np.float32)
        kc = np.clip(kf, -126, 127).astype(np.int32)
        two_k = ((kc + 127).astype(np.uint32) << np.uint32(23)).view(np.float32)
        y = (p * two_k).astype(np.float32)
    y = np.where(x < EXP_LO, f32(0.0), y)
    y = np.where(x > EXP_HI, f32(np.inf), y)
    return y.astype(np.float32)


def tree_sum_f32(t: np.ndarray) -> np.ndarray:
    """Sum along the last axis in float32 by a halving-stride binary tree over
    the axis zero-padded to a power of two: pass s adds element i+s to i."""
    t = np.asarray(t, dtype=np.float32)
    E = t.shape[-1]
    P = 1
    while P < E:
        P *= 2
    pad = np.zeros(t.shape[:-1] + (P,), dtype=np.float32)
    pad[..., :E] = t
    s = P // 2
    while s >= 1:
        pad[..., :s] = pad[..., :s] + pad[..., s:2 * s]
        s //= 2
    return pad[..., 0].astype(np.float32)


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Specified softmax over the expert axis: shift by the row max, spec_exp,
    tree sum, IEEE division (page 2: S = softmax(X W_g))."""
    z = np.asarray(z, dtype=np.float32)
    m = z.max(axis=-1, keepdims=True)
    t = spec_exp(z - m)
    s = tree_sum_f32(t)[..., None]
    return (t / s).astype(np.float32)


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Specified sigmoid 1 / (1 + spec_exp(-z)) (page 5 strategy 4: DeepSeek-V3
    gives every expert its own sigmoid score in place of a softmax row)."""
    z = np.asarray(z, dtype=np.float32)
    with np.errstate(over="ignore", divide="ignore"):
        return (f32(1.0) / (f32(1.0) + spec_exp(-z))).astype(np.float32)


# Specified float32 log1p on [0, 1]: log1p(u) = 2 atanh(s), s = u / (2 + u),
# and 2 atanh(s) = 2 s (1 + s^2/3 + s^4/5 + ... + s^14/15).  For u in [0, 1],
# s <= 1/3, so the first omitted term is below (1/9)^8 / 17 < 2^-30 relative.
# The series runs in Horner form over s^2 with float32 coefficients 1/(2j+1).
LOG1P_COEF = [f32(1.0 / (2 * j + 1)) for j in range(8)]        # 1/1, 1/3, ..., 1/15


def spec_log1p(u) -> np.ndarray:
    """Specified float32 log(1 + u) for 0 <= u <= 1; one IEEE float32
    operation per step."""
    u = np.asarray(u, dtype=np.float32)
    s = (u / (f32(2.0) + u)).astype(np.float32)
    s2 = (s * s).astype(np.float32)
    p = LOG1P_COEF[7]
    for j in range(6, -1, -1):
        p = (p * s2 + LOG1P_COEF[j]).astype(np.float32)
    return ((s + s) * p).astype(np.float32)


def spec_softplus(z) -> np.ndarray:
    """Specified float32 softplus log(1 + e^z) = max(z, 0) + log1p(e^-|z|)."""
    z = np.asarray(z, dtype=np.float32)
    return (np.maximum(z, f32(0.0)) + spec_log1p(spec_exp(-np.abs(z)))).astype(np.float32)


def sqrtsoftplus(z) -> np.ndarray:
    """Specified sqrtsoftplus score sqrt(softplus(z)) with the correctly rounded
    float32 square root (page 5 strategy 4: DeepSeek-V4 scores experts with
    sqrtsoftplus and keeps the bias balancing of the sigmoid recipe)."""
    return np.sqrt(spec_softplus(z)).astype(np.float32)


def expert_score(z: np.ndarray, score: str) -> np.ndarray:
    """Per-expert score of the bias-balanced recipes: sigmoid or sqrtsoftplus."""
    if score == "sigmoid":
        return sigmoid(z)
    if score == "sqrtsoftplus":
        return sqrtsoftplus(z)
    raise ValueError(score)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, wg: np.ndarray, logit_offset: Optional[np.ndarray] = None,
                  noise: Optional[np.ndarray] = None, noise_std: float = 0.0):
    """Z = X W_g with W_g in the pages' [d, E] layout (page 2 "Token-choice
    ...": s = softmax(x W_g), W_g: [d, E]); the product is exact-ish in
    float64 and rounded once to float32; a per-expert offset is then added in
    float32.  Noisy top-k (page 4 "Pitfalls": Gaussian noise added to the
    gating logits) adds noise_std * noise[t, e] last, with the standard
    normals `noise` drawn by the caller: one float32 multiply, one add."""
    z = (widen(x) @ widen(wg)).astype(np.float32)
    if logit_offset is not None:
        z = (z + np.asarray(logit_offset, dtype=np.float32)[None, :]).astype(np.float32)
    if noise is not None:
        z = (z + (f32(noise_std) * np.asarray(noise, dtype=np.float32))).astype(np.float32)
    return z


def router_scores(z: np.ndarray, score: str) -> np.ndarray:
    return softmax_rows(z) if score == "softmax" else expert_score(z, score)


# ---------------------------------------------------------------------------
# Sizes
# ---------------------------------------------------------------------------


def round_half_up(v: float) -> int:
    return int(math.floor(v + 0.5))


def ec_k(n: int, c: float, E: int) -> int:
    """Tokens per expert under expert choice, k = n c / E (page 1 "Who picks
    whom"; page 2 "A worked example"), rounded half up when not integral."""
    return round_half_up(n * c / E)


def tc_capacity(n: int, k: int, E: int, cf: Optional[float]) -> int:
    """Per-expert buffer under token choice: cf * (balanced load n k / E).
    For k = 1 this is page 5's tokens-per-batch / experts x capacity factor;
    for k > 1 the balanced load n k / E is page 1's one-eighth-of-the-tokens
    share at 8 of 64.  None (dropless) -> unlimited (returned as n*k)."""
    if cf is None:
        return n * k
    return round_half_up(cf * k * n / E)


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------


def _stable_desc_order(keys: np.ndarray, axis: int) -> np.ndarray:
    """Indices sorting `keys` in descending order along `axis`, equal keys in
    ascending index order (a stable sort of the negated keys)."""
    with np.errstate(invalid="ignore"):
        return np.argsort(-keys, axis=axis, kind="stable")


def group_mask(keys: np.ndarray, n_group: int, topk_group: int, topm: int) -> np.ndarray:
    """Group-limited pre-selection (page 5 strategy 5): experts form n_group
    contiguous groups; each group is scored by the sum of its top-`topm` keys
    (topm = 1: its highest key), summed in float32 in descending order; the
    `topk_group` best groups are kept (lowest group index first on ties).
    Returns a boolean [n, E] mask of experts in kept groups."""
    n, E = keys.shape
    gsz = E // n_group
    kg = keys.reshape(n, n_group, gsz)
    srt = np.take_along_axis(kg, _stable_desc_order(kg, axis=2), axis=2)
    gscore = srt[:, :, 0].astype(np.float32)
    for j in range(1, topm):
        gscore = (gscore + srt[:, :, j]).astype(np.float32)
    gorder = _stable_desc_order(gscore, axis=1)[:, :topk_group]
    keep_g = np.zeros((n, n_group), dtype=bool)
    np.put_along_axis(keep_g, gorder, True, axis=1)
    return np.repeat(keep_g, gsz, axis=1)


def select_token_choice(z: np.ndarray, k: int, score: str = "softmax",
                        sel_bias: Optional[np.ndarray] = None, n_group: int = 1,
                        topk_group: int = 1, topm: int = 1, norm_topk: bool = True):
    """Token choice: every token keeps its k best experts.

    Keys: softmax scoring selects on the logits themselves (softmax is
    monotone within a row, and page 3 selects on z_t directly); sigmoid (or
    sqrtsoftplus) scoring selects on score(z) + b, the bias entering the
    choice only (page 5 strategy 4).  Optional group-limited pre-selection.  Equal keys:
    the lower expert index wins.

    Gates (mixing weights):
      softmax, norm_topk: softmax over the k selected logits (page 5 strategy
        1), i.e. t_j = spec_exp(z_j - z_top), w_j = t_j / (t_0 + ... + t_{k-1})
        summed left to right in rank order;
      softmax, not norm_topk: the full-row softmax probability p_e (the
        top-1 Switch gate);
      sigmoid / sqrtsoftplus: raw scores (no bias), renormalised over the k
        when norm_topk (page 5 strategy 4: mixing weights from the raw
        scores).
    Returns idx [n, k] int32 in rank order and gate [n, k] float32.
    """
    z = np.asarray(z, dtype=np.float32)
    n, E = z.shape
    if score == "softmax":
        keys = z.copy()
    else:
        sig = expert_score(z, score)
        keys = sig if sel_bias is None else (sig + np.asarray(sel_bias, np.float32)[None, :])
        keys = keys.astype(np.float32)
    if n_group > 1:
        keys = np.where(group_mask(keys, n_group, topk_group, topm), keys, f32(-np.inf))
    idx = _stable_desc_order(keys, axis=1)[:, :k].astype(np.int32)

    if score == "softmax":
        if norm_topk:
            zs = np.take_along_axis(z, idx, axis=1)
            t = spec_exp((zs - zs[:, :1]).astype(np.float32))
            s = t[:, 0].copy()
            for j in range(1, k):
                s = (s + t[:, j]).astype(np.float32)
            gate = (t / s[:, None]).astype(np.float32)
        else:
            gate = np.take_along_axis(softmax_rows(z), idx, axis=1)
    else:
        raw = np.take_along_axis(expert_score(z, score), idx, axis=1)
        if norm_topk:
            s = raw[:, 0].copy()
            for j in range(1, k):
                s = (s + raw[:, j]).astype(np.float32)
            gate = (raw / s[:, None]).astype(np.float32)
        else:
            gate = raw
    return idx, gate.astype(np.float32)


def select_expert_choice(z: np.ndarray, k: int):
    """Expert choice (page 2 "The math": G, I = TopK(S^T, k) over the token
    axis): every expert keeps the k tokens with the highest softmax score in
    its column; equal scores -> lower token index.  I[e] is returned in
    ascending token order (the layer's result does not depend on the order
    within I[e]); G[e, j] = S[I[e, j], e]."""
    S = softmax_rows(z)
    n, E = S.shape
    order = _stable_desc_order(S, axis=0)[:k, :]          # [k, E]
    I = np.sort(order, axis=0).T.astype(np.int32)         # [E, k]
    G = S[I, np.arange(E)[:, None]].astype(np.float32)
    return I, G


# ---------------------------------------------------------------------------
# Routing map
# ---------------------------------------------------------------------------


def build_map_token_choice(idx: np.ndarray, gate: np.ndarray, E: int, capacity: Optional[int],
                           order: str = "token"):
    """Literal sequential arrival loop (page 1: tokens that arrive after an
    expert's buffer fills skip it; page 5 strategy 2).  order "token": the
    assignments arrive in token order, and within a token in rank order;
    order "rank": every token's first choice arrives before any second
    choice (rank-major priority), tokens in order within a rank.  An
    assignment is kept iff fewer than `capacity` earlier arrivals went to the
    same expert (capacity None = dropless).  Kept assignments occupy compact
    expert-major slots in arrival order."""
    n, k = idx.shape
    if order == "token":
        arrivals = [(t, r) for t in range(n) for r in range(k)]
    elif order == "rank":
        arrivals = [(t, r) for r in range(k) for t in range(n)]
    else:
        raise ValueError(order)
    C = n * k if capacity is None else int(capacity)
    count = np.bincount(idx.reshape(-1), minlength=E).astype(np.int64)
    kept = np.minimum(count, C)
    offset = np.zeros(E + 1, dtype=np.int64)
    offset[1:] = np.cumsum(kept)
    M = int(offset[-1])
    slot_token = np.empty(M, dtype=np.int32)
    slot_gate = np.empty(M, dtype=np.float32)
    assign_slot = np.full((n, k), -1, dtype=np.int32)
    fill = [0] * E
    idx_l = idx.tolist()
    gate_l = gate.tolist()
    off_l = offset.tolist()
    for t, r in arrivals:
        e = idx_l[t][r]
        pos = fill[e]
        fill[e] = pos + 1
        if pos < C:
            s = off_l[e] + pos
            slot_token[s] = t
            slot_gate[s] = gate_l[t][r]
            assign_slot[t, r] = s
    # token-side lists: token t's k assignments in rank order, -1 where dropped
    token_offset = (np.arange(n + 1, dtype=np.int64) * k).astype(np.int32)
    token_slot = assign_slot.reshape(-1).copy()
    return dict(expert_count=count.astype(np.int32), expert_offset=offset.astype(np.int32),
                slot_token=slot_token, slot_gate=slot_gate, assign_slot=assign_slot,
                token_offset=token_offset, token_slot=token_slot, n_kept=M)


def build_map_expert_choice(I: np.ndarray, G: np.ndarray, n: int):
    """Expert choice needs no capacity: expert e owns slots e*k .. e*k+k-1 in
    the order of I[e].  Token-side lists run in ascending expert order."""
    E, k = I.shape
    slot_token = I.reshape(-1).astype(np.int32)
    slot_gate = G.reshape(-1).astype(np.float32)
    assign_slot = (np.arange(E * k, dtype=np.int32)).reshape(E, k)
    count = np.full(E, k, dtype=np.int32)
    offset = (np.arange(E + 1, dtype=np.int64) * k).astype(np.int32)
    per_tok = [[] for _ in range(n)]
    for e in range(E):                       # ascending expert order
        for j in range(k):
            per_tok[int(I[e, j])].append(e * k + j)
    token_offset = np.zeros(n + 1, dtype=np.int64)
    token_offset[1:] = np.cumsum([len(p) for p in per_tok])
    token_slot = np.array([s for p in per_tok for s in p], dtype=np.int32)
    return dict(expert_count=count, expert_offset=offset, slot_token=slot_token,
                slot_gate=slot_gate, assign_slot=assign_slot,
                token_offset=token_offset.astype(np.int32), token_slot=token_slot, n_kept=E * k)


# ---------------------------------------------------------------------------
# Dispatch, experts, combine
# ---------------------------------------------------------------------------


def dispatch(x: np.ndarray, slot_token: np.ndarray) -> np.ndarray:
    """X_in = P X: row s of the expert-major buffer is token slot_token[s]."""
    return x[slot_token]


def gelu(h: np.ndarray) -> np.ndarray:
    """Exact GELU, x * Phi(x) = x/2 (1 + erf(x / sqrt 2))."""
    from scipy.special import erf
    return 0.5 * h * (1.0 + erf(h / math.sqrt(2.0)))


def silu(h: np.ndarray) -> np.ndarray:
    return h / (1.0 + np.exp(-h))


def expert_hidden(xe: np.ndarray, w1: np.ndarray, act: str) -> np.ndarray:
    """The expert's hidden activation in float64: GELU: gelu(x W1^T);
    SwiGLU: silu(x Wg^T) * (x Wu^T) with W1 = [Wg; Wu] (gate rows first)."""
    x = widen(xe) if xe.dtype == np.uint16 else np.asarray(xe, dtype=np.float64)
    W1 = widen(w1)
    if act == "gelu":
        return gelu(x @ W1.T)
    f = W1.shape[0] // 2
    return silu(x @ W1[:f].T) * (x @ W1[f:].T)


def expert_forward(xe: np.ndarray, w1: np.ndarray, w2: np.ndarray, act: str) -> np.ndarray:
    """One expert FFN in float64: hidden activation, then h W2^T."""
    return expert_hidden(xe, w1, act) @ widen(w2).T


def expert_ffn(x_perm: np.ndarray, expert_offset: np.ndarray, w1_of, w2_of, act: str,
               experts=None) -> np.ndarray:
    """Grouped FFN over the expert-major buffer: rows offset[e]..offset[e+1]
    go through expert e.  w1_of(e) / w2_of(e) return expert e's weights (so a
    caller can stream one expert at a time).  `experts` limits the experts
    evaluated (others' rows stay zero)."""
    M = int(expert_offset[-1])
    d = x_perm.shape[1]
    y = np.zeros((M, d), dtype=np.float64)
    E = len(expert_offset) - 1
    for e in (range(E) if experts is None else experts):
        a, b = int(expert_offset[e]), int(expert_offset[e + 1])
        if b > a:
            y[a:b] = expert_forward(x_perm[a:b], w1_of(e), w2_of(e), act)
    return y


def combine(y_perm: np.ndarray, slot_gate: np.ndarray, token_offset: np.ndarray,
            token_slot: np.ndarray, n: int, residual: Optional[np.ndarray] = None,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """out = scatter_add(G * Y, I) (page 2 "The math"): each token sums its
    experts' gate-weighted outputs (gate applied to the expert output), plus
    the always-on shared expert and the residual; a token with no kept expert
    keeps the residual alone (page 1; page 2 "Variable tokens-per-token")."""
    d = y_perm.shape[1]
    branch = np.zeros((n, d), dtype=np.float64)
    for t in range(n):
        for q in range(int(token_offset[t]), int(token_offset[t + 1])):
            s = int(token_slot[q])
            if s >= 0:                          # -1: an assignment dropped at capacity
                branch[t] += float(slot_gate[s]) * y_perm[s]
    out = branch
    if shared is not None:
        out = out + np.asarray(shared, dtype=np.float64)
    if residual is not None:
        out = out + (widen(residual) if residual.dtype == np.uint16 else residual.astype(np.float64))
    return out


# ---------------------------------------------------------------------------
# Balance statistics
# ---------------------------------------------------------------------------
STAT_NAMES = ("lb_loss", "z_loss", "max_vio", "max_load_share", "n_kept", "n_dropped",
              "tokens_without_expert", "max_experts_per_token")


def balance_stats(z: np.ndarray, rmap: dict, direction: str, k: int, score: str,
                  lb_coef: float, z_coef: float):
    """Routing health numbers (page 1 "What each direction guarantees"; page
    4 "Pitfalls"; page 5 TL;DR).  Readings:

    lb_loss = coef * E * sum_e f_e P_e, f_e = chosen_e / sum(chosen) (before
              drops), P_e = mean over tokens of the normalised score
              (softmax probability; for sigmoid or sqrtsoftplus scores the
              score / its row sum);
              equals coef exactly at a balanced load.
    z_loss  = coef * mean_t (logsumexp_e z_te)^2.
    max_vio = (max_e load_e - mean_e load_e) / mean_e load_e, load = kept
              assignments per expert.
    max_load_share = max_e load_e / sum_e load_e (collapse flag).
    Also kept and dropped assignments, tokens with no kept expert, the most
    experts any token has, and the experts-per-token histogram [E+1].
    """
    z64 = np.asarray(z, dtype=np.float64)
    n, E = z64.shape
    count = rmap["expert_count"].astype(np.float64)
    load = np.diff(rmap["expert_offset"].astype(np.int64)).astype(np.float64)
    f = count / count.sum() if count.sum() > 0 else np.zeros_like(count)   # nothing chosen: f = 0
    if score == "softmax":
        zm = z64 - z64.max(axis=1, keepdims=True)
        p = np.exp(zm) / np.exp(zm).sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        sg = 1.0 / (1.0 + np.exp(-z64))
        p = sg / sg.sum(axis=1, keepdims=True)
    else:
        sg = np.sqrt(np.logaddexp(0.0, z64))                 # sqrt(softplus(z)) in float64
        p = sg / sg.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    lb = lb_coef * E * float((f * P).sum())
    m = z64.max(axis=1)
    lse = m + np.log(np.exp(z64 - m[:, None]).sum(axis=1))
    zl = z_coef * float((lse ** 2).mean())
    mean_load = load.mean()
    max_vio = float((load.max() - mean_load) / mean_load) if mean_load > 0 else 0.0
    n_kept = int(rmap["n_kept"])
    total = n * k if direction == "tc" else E * k
    kept_entry = (rmap["token_slot"] >= 0).astype(np.int64)
    per_tok = np.array([kept_entry[a:b].sum() for a, b in
                        zip(rmap["token_offset"][:-1], rmap["token_offset"][1:])], dtype=np.int64)
    hist = np.bincount(per_tok, minlength=E + 1)[:E + 1].astype(np.int64)
    stats = np.array([lb, zl, max_vio, float(load.max()) / max(n_kept, 1), n_kept,
                      total - n_kept, int((per_tok == 0).sum()), int(per_tok.max(initial=0))],
                     dtype=np.float64)
    return stats, hist


def update_bias(bias: np.ndarray, expert_count: np.ndarray, n: int, k: int, gamma: float):
    """Auxiliary-loss-free balancing step (page 5 strategy 4: once per step,
    the bias of an over-used expert goes down and that of an under-used one
    up).  Reading:
    load_e = assignments chosen for expert e this step (before capacity
    drops), mean = n k / E; b_e <- b_e - gamma * sign(load_e - mean), with the
    sign taken exactly in integers (sign(load_e * E - n * k)), so an expert
    exactly at the mean keeps its bias.  One float32 subtraction per expert."""
    b = np.asarray(bias, dtype=np.float32)
    E = b.shape[0]
    diff = np.asarray(expert_count, dtype=np.int64) * E - int(n) * int(k)
    step = (f32(gamma) * np.sign(diff).astype(np.float32)).astype(np.float32)
    return (b - step).astype(np.float32)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------


def forward(cfg, inp: dict, inject_logits: Optional[np.ndarray] = None, experts=None,
            w1_of=None, w2_of=None, residual: bool = True):
    """The layer forward, stage by stage.  `cfg` needs the MoEConfig fields
    (n, d, E, k | c, f, act, direction, score, capacity_factor, norm_topk,
    n_group, topk_group, group_topm, shared_f, lb_coef, z_coef); `inp` the
    arrays x, wg, logit_offset, sel_bias, w1, w2 (or w1_of / w2_of callables),
    shared_w1, shared_w2.  With `inject_logits` the selection and everything
    after it run on those float32 logits (so a caller can compare against a
    device whose logits differ in the last bits).  Returns a dict of every
    stage's result."""
    x = inp["x"]
    z_ref = router_logits(x, inp["wg"], inp.get("logit_offset"), inp.get("noise"),
                          getattr(cfg, "noise_std", 0.0))
    z = z_ref if inject_logits is None else np.asarray(inject_logits, dtype=np.float32)
    n, E = z.shape
    res = dict(logits=z_ref)
    if cfg.direction == "tc":
        k = cfg.k
        idx, gate = select_token_choice(z, k, cfg.score, inp.get("sel_bias"), cfg.n_group,
                                        cfg.topk_group, cfg.group_topm, cfg.norm_topk)
        cap = tc_capacity(n, k, E, cfg.capacity_factor)
        rmap = build_map_token_choice(idx, gate, E, None if cfg.capacity_factor is None else cap,
                                      getattr(cfg, "capacity_order", "token"))
        res.update(sel_idx=idx, sel_gate=gate, capacity=cap)
    else:
        k = ec_k(n, cfg.c, E)
        I, G = select_expert_choice(z, k)
        rmap = build_map_expert_choice(I, G, n)
        res.update(sel_idx=I, sel_gate=G)
    res["k"] = k
    res["map"] = rmap
    x_perm = dispatch(x, rmap["slot_token"])
    res["x_perm"] = x_perm
    w1_of = w1_of or (lambda e: inp["w1"][e])
    w2_of = w2_of or (lambda e: inp["w2"][e])
    y_perm = expert_ffn(x_perm, rmap["expert_offset"], w1_of, w2_of, cfg.act, experts)
    res["y_perm"] = y_perm
    shared = None
    if cfg.shared_f:
        shared = expert_forward(x, inp["shared_w1"], inp["shared_w2"], cfg.act)
        res["shared"] = shared
    res["branch"] = combine(y_perm, rmap["slot_gate"], rmap["token_offset"], rmap["token_slot"], n,
                            None, shared)
    res["out"] = combine(y_perm, rmap["slot_gate"], rmap["token_offset"], rmap["token_slot"], n,
                         x if residual else None, shared)
    res["stats"], res["hist"] = balance_stats(z, rmap, cfg.direction, k, cfg.score,
                                              cfg.lb_coef, cfg.z_coef)
    return res


def forward_dense(cfg, inp: dict, z: np.ndarray, residual: bool = True) -> np.ndarray:
    """Second, independent formulation of the same layer: no permutation at
    all.  Every expert runs on every token; the result is the sum over
    experts of (one-hot keep mask) * gate * FFN_e(x), the mask being built
    from the selection by cumulative counts instead of the arrival loop.  The
    oracle's gather/scatter path must agree with it."""
    x = inp["x"]
    n, E = z.shape
    W = np.zeros((n, E), dtype=np.float64)          # dense gate-times-keep matrix
    if cfg.direction == "tc":
        k = cfg.k
        idx, gate = select_token_choice(z, k, cfg.score, inp.get("sel_bias"), cfg.n_group,
                                        cfg.topk_group, cfg.group_topm, cfg.norm_topk)
        # arrivals as rows of a one-hot matrix, in token-major or rank-major order
        seq = idx if getattr(cfg, "capacity_order", "token") == "token" else idx.T
        onehot = np.zeros((n * k, E), dtype=np.int64)
        onehot[np.arange(n * k), seq.reshape(-1)] = 1
        before = np.cumsum(onehot, axis=0) - onehot          # earlier arrivals per expert
        pos = before[np.arange(n * k), seq.reshape(-1)].reshape(seq.shape)
        if seq is not idx:
            pos = pos.T
        C = n * k if cfg.capacity_factor is None else tc_capacity(n, k, E, cfg.capacity_factor)
        keep = pos < C
        for r in range(k):
            W[np.arange(n), idx[:, r]] += np.where(keep[:, r], gate[:, r].astype(np.float64), 0.0)
    else:
        k = ec_k(n, cfg.c, E)
        I, G = select_expert_choice(z, k)
        for e in range(E):
            W[I[e], e] = G[e].astype(np.float64)
    out = np.zeros((n, x.shape[1]), dtype=np.float64)
    for e in range(E):
        if np.any(W[:, e] != 0):
            out += W[:, e:e + 1] * expert_forward(x, inp["w1"][e], inp["w2"][e], cfg.act)
    if cfg.shared_f:
        out += expert_forward(x, inp["shared_w1"], inp["shared_w2"], cfg.act)
    if residual:
        out += widen(x) if x.dtype == np.uint16 else x.astype(np.float64)
    return out
