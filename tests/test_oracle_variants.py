"""Pins of the oracle's routing variants against facts from outside the
oracle: float64 references of the specified float32 functions, brute-force
enumeration, hand-worked maps, closed forms and the direction of the
balancing feedback.

Variants (page 5 "MoE routing strategies explained", strategy 4; page 4
"How MoE routing strategies make LLMs efficient", section "Pitfalls"):
sqrtsoftplus expert scores, the auxiliary-loss-free bias update, Gaussian
noise on the gating logits, and rank-major capacity priority (the other
arrival order for the capacity rule of page 1 "Dropped tokens flow in
opposite directions")."""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from test_oracle_pins import dominant_subset, ulp_distance


# ---------------------------------------------------------------- specified functions

def test_spec_log1p_faithful_to_float64():
    rng = np.random.default_rng(21)
    u = np.concatenate([np.linspace(0, 1, 1_000_001, dtype=np.float32),
                        rng.uniform(0, 1, 300_000).astype(np.float32),
                        (10.0 ** rng.uniform(-30, -1, 100_000)).astype(np.float32)])
    got = O.spec_log1p(u)
    ref = np.log1p(u.astype(np.float64)).astype(np.float32)
    d = ulp_distance(got, ref)
    assert d.max() <= 3, f"max ulp {d.max()} at u={u[d.argmax()]}"
    assert O.spec_log1p(np.float32(0.0)) == 0.0
    assert ulp_distance(O.spec_log1p(np.float32(1.0)), np.float32(math.log(2.0))) <= 1
    tiny = np.float32([1e-30, 1e-20, 1e-12, 3e-8])
    assert (ulp_distance(O.spec_log1p(tiny), tiny) <= 1).all()      # log1p(u) = u for tiny u


def test_spec_softplus_faithful_and_closed_forms():
    z = np.linspace(-80, 80, 1_600_001, dtype=np.float32)
    got = O.spec_softplus(z)
    ref = np.logaddexp(0.0, z.astype(np.float64)).astype(np.float32)
    d = ulp_distance(got, ref)
    assert d.max() <= 4, f"max ulp {d.max()} at z={z[d.argmax()]}"
    assert ulp_distance(O.spec_softplus(np.float32(0.0)), np.float32(math.log(2.0))) <= 1
    # softplus(z) - softplus(-z) = z
    zz = np.linspace(0, 30, 30001, dtype=np.float32)
    diff = O.spec_softplus(zz).astype(np.float64) - O.spec_softplus(-zz).astype(np.float64)
    assert np.abs(diff - zz).max() <= 4 * np.spacing(np.float32(30.0))
    # far right: exactly z (e^-|z| is flushed to 0 below -86); far left: 0
    big = np.float32([86.5, 100.0, 1e6])
    assert np.array_equal(O.spec_softplus(big), big)
    assert O.spec_softplus(np.float32(-90.0)) == 0.0


def test_sqrtsoftplus_faithful_and_monotone():
    z = np.linspace(-80, 80, 1_600_001, dtype=np.float32)
    got = O.sqrtsoftplus(z)
    ref = np.sqrt(np.logaddexp(0.0, z.astype(np.float64))).astype(np.float32)
    d = ulp_distance(got, ref)
    assert d.max() <= 3, f"max ulp {d.max()} at z={z[d.argmax()]}"
    assert (np.diff(got.astype(np.float64)) >= 0).all()
    assert ulp_distance(O.sqrtsoftplus(np.float32(0.0)), np.float32(math.sqrt(math.log(2.0)))) <= 1
    assert (O.sqrtsoftplus(z) >= 0).all()


# ---------------------------------------------------------------- sqrtsoftplus selection

def test_sqrtsoftplus_selection_brute_force():
    rng = np.random.default_rng(22)
    for (E, ng, tg, topm, k) in ((8, 1, 1, 1, 3), (8, 4, 2, 1, 3), (8, 2, 1, 2, 2), (6, 3, 2, 1, 4)):
        z = rng.normal(size=(60, E)).astype(np.float32)
        z[:10] = np.round(z[:10])                               # ties
        b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
        idx, gate = O.select_token_choice(z, k, "sqrtsoftplus", b, ng, tg, topm, True)
        keys = (O.sqrtsoftplus(z) + b[None]).astype(np.float32)
        gsz = E // ng
        for t in range(z.shape[0]):
            kt = keys[t].tolist()
            if ng > 1:
                gs = []
                for g in range(ng):
                    v = sorted(kt[g * gsz:(g + 1) * gsz], reverse=True)
                    s = np.float32(v[0])
                    for j in range(1, topm):
                        s = np.float32(s + np.float32(v[j]))
                    gs.append(float(s))
                kept = dominant_subset(gs, tg)
                kt = [kt[e] if e // gsz in kept else -math.inf for e in range(E)]
            assert set(idx[t].tolist()) == dominant_subset(kt, k)
        # gates: the raw scores of the chosen experts, renormalised (no bias)
        raw = np.take_along_axis(np.sqrt(np.logaddexp(0.0, z.astype(np.float64))), idx, 1)
        assert np.abs(gate - raw / raw.sum(1, keepdims=True)).max() < 2e-6


def test_sqrtsoftplus_without_bias_keeps_the_largest_logits():
    # the score is increasing in z, so with no bias and well separated logits
    # the choice is the plain top-k of the logits
    rng = np.random.default_rng(23)
    z = np.stack([rng.permutation(16) * 0.37 - 3.0 for _ in range(50)]).astype(np.float32)
    a, _ = O.select_token_choice(z, 4, "sqrtsoftplus", None, norm_topk=True)
    b, _ = O.select_token_choice(z, 4, "softmax", None, norm_topk=True)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- rank-major capacity

def test_map_hand_example_rank_order():
    # the token-order hand example, rank-major: arrivals are the first
    # choices (t0:e0, t1:e1, t2:e0) then the second ones (t0:e1, t1:e0,
    # t2:e1).  Capacity 2: expert 0 keeps t0 and t2 and drops t1's second
    # choice; expert 1 keeps t1 and t0 and drops t2's second choice.  Every
    # token keeps its first choice (token order dropped token 2 entirely).
    idx = np.int32([[0, 1], [1, 0], [0, 1]])
    gate = np.float32([[0.6, 0.4], [0.7, 0.3], [0.5, 0.5]])
    m = O.build_map_token_choice(idx, gate, 2, 2, order="rank")
    assert m["expert_count"].tolist() == [3, 3]
    assert m["expert_offset"].tolist() == [0, 2, 4]
    assert m["slot_token"].tolist() == [0, 2, 1, 0]
    assert m["assign_slot"].tolist() == [[0, 3], [2, -1], [1, -1]]
    assert m["token_offset"].tolist() == [0, 2, 4, 6]
    assert m["token_slot"].tolist() == [0, 3, 2, -1, 1, -1]
    assert np.allclose(m["slot_gate"], [0.6, 0.5, 0.7, 0.4])


def test_map_rank_order_brute_force():
    rng = np.random.default_rng(24)
    for (n, E, k, C) in ((50, 4, 2, 20), (64, 8, 3, 10), (30, 3, 1, 5), (40, 5, 2, 1000)):
        z = rng.normal(size=(n, E)).astype(np.float32)
        z[:, 0] += 1.0
        idx, gate = O.select_token_choice(z, k, "softmax", norm_topk=True)
        m = O.build_map_token_choice(idx, gate, E, C, order="rank")
        arrivals = [(t, r, int(idx[t, r])) for r in range(k) for t in range(n)]
        for e in range(E):
            mine = [(t, r) for (t, r, ee) in arrivals if ee == e]
            a, b = m["expert_offset"][e], m["expert_offset"][e + 1]
            assert b - a == min(len(mine), C)
            assert m["slot_token"][a:b].tolist() == [t for t, _ in mine[:C]]
            for (t, r) in mine[C:]:
                assert m["assign_slot"][t, r] == -1
            # priority: a kept choice of rank r implies every lower-rank choice of e is kept
            kept_r = [r for (t, r) in mine[:C]]
            dropped_r = [r for (t, r) in mine[C:]]
            if kept_r and dropped_r:
                assert max(kept_r) <= min(dropped_r)
        mt = O.build_map_token_choice(idx, gate, E, C, order="token")
        if k == 1:
            for key in ("expert_offset", "slot_token", "assign_slot", "token_slot"):
                assert np.array_equal(m[key], mt[key])
        if C >= n * k:      # dropless: same kept set, slots in a different order
            assert (m["assign_slot"] >= 0).all() and (mt["assign_slot"] >= 0).all()


# ---------------------------------------------------------------- bias update

def test_update_bias_closed_forms():
    b = np.float32([0.5, -0.25, 0.0, 1e-3])
    # balanced: every expert exactly at the mean keeps its bias
    assert np.array_equal(O.update_bias(b, np.int32([5, 5, 5, 5]), 10, 2, 0.01), b)
    # over / under / at the mean: one float32 step of gamma each way
    got = O.update_bias(b, np.int32([7, 3, 5, 5]), 10, 2, 0.01)
    want = np.float32([np.float32(0.5) - np.float32(0.01), np.float32(-0.25) + np.float32(0.01), 0.0, 1e-3])
    assert np.array_equal(got, want)
    # fractional mean (3 tokens, 2 experts): 2 > 1.5 > 1
    got = O.update_bias(np.float32([0.0, 0.0]), np.int32([2, 1]), 3, 1, 0.125)
    assert got.tolist() == [-0.125, 0.125]
    assert np.array_equal(O.update_bias(b, np.int32([9, 0, 1, 10]), 10, 2, 0.0), b)


def test_bias_feedback_balances_a_skewed_router():
    # a fixed router with a strong per-expert preference; repeated steps of
    # the update must drive the load toward the mean (the pages report
    # MaxVio falling with loss-free balancing).  A flipped sign would make
    # the skew worse.
    rng = np.random.default_rng(25)
    n, E, k = 2000, 16, 2
    z = (rng.normal(size=(n, E)) - 1.1 * np.log(np.arange(1, E + 1))[None, :]).astype(np.float32)
    b = np.zeros(E, np.float32)

    def max_vio(bias):
        idx, _ = O.select_token_choice(z, k, "sigmoid", bias, norm_topk=True)
        cnt = np.bincount(idx.reshape(-1), minlength=E)
        return cnt, (cnt.max() - cnt.mean()) / cnt.mean()

    cnt, v0 = max_vio(b)
    for _ in range(300):
        b = O.update_bias(b, cnt, n, k, 0.002)
        cnt, v = max_vio(b)
    assert v0 > 1.0 and v < 0.15 * v0, (v0, v)


# ---------------------------------------------------------------- noisy logits

def test_noise_enters_the_logits_last():
    rng = np.random.default_rng(26)
    x = rng.normal(size=(20, 32)).astype(np.float32)
    wg = (rng.normal(size=(32, 8)) / 6).astype(np.float32)
    off = rng.normal(size=8).astype(np.float32)
    eps = rng.standard_normal((20, 8)).astype(np.float32)
    z = O.router_logits(x, wg, off)
    assert np.array_equal(O.router_logits(x, wg, off, eps, 0.0), z)       # zero scale: no change
    zn = O.router_logits(x, wg, off, eps, 1.5)
    assert np.array_equal(zn, (z + np.float32(1.5) * eps).astype(np.float32))
    # a large draw on one expert forces it into every token's choice
    spike = np.zeros((20, 8), np.float32)
    spike[:, 6] = 1e3
    idx, _ = O.select_token_choice(O.router_logits(x, wg, off, spike, 1.0), 2, "softmax")
    assert (idx[:, 0] == 6).all()
