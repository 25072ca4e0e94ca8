"""CPU checks of the derived bf16 error bound (tests/bounds.py): a numpy
emulation of the device's rounding points stays inside it, and plausible
mistakes (a dropped K block of the down projection, a wrong row, a scaled
output, a missing expert in the branch) fall outside it."""
import numpy as np
import pytest

from bounds import BranchBound, ExpertRows, check_branch, check_rows
from oracle import moe_oracle as O
from sparse_expert_dispatch_amd.workloads import f32_to_bf16_bits


def bits_to_f32(a):
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def emulate_device(xe, w1, w2, act, drop_k=None):
    """The device's rounding points in numpy: fp32 pre-activation, fp32
    activation, H rounded to bf16, fp32 down projection, Y rounded to bf16.
    drop_k: a slice of the down projection's K left out (a planted bug)."""
    x, W1, W2 = bits_to_f32(xe), bits_to_f32(w1), bits_to_f32(w2)
    A = (x @ W1.T).astype(np.float32)
    f = W2.shape[1]
    if act == "gelu":
        h = O.gelu(A.astype(np.float64)).astype(np.float32)
    else:
        g, u = A[:, :f].astype(np.float64), A[:, f:].astype(np.float64)
        h = (O.silu(g) * u).astype(np.float32)
    hb = bits_to_f32(f32_to_bf16_bits(h))
    if drop_k is not None:
        hb = hb.copy()
        hb[:, drop_k] = 0
    y = (hb @ W2.T).astype(np.float32)
    return f32_to_bf16_bits(y)


def make(act, m, d, f, seed):
    rng = np.random.default_rng(seed)
    rows = 2 * f if act == "swiglu" else f
    xe = f32_to_bf16_bits(rng.standard_normal((m, d), dtype=np.float32))
    w1 = f32_to_bf16_bits((rng.standard_normal((rows, d)) / np.sqrt(d)).astype(np.float32))
    w2 = f32_to_bf16_bits((rng.standard_normal((d, f)) / np.sqrt(f)).astype(np.float32))
    return xe, w1, w2


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_emulated_device_rows_within_bound(act):
    xe, w1, w2 = make(act, 96, 256, 512, 1)
    R = ExpertRows(xe, w1, w2, act)
    err = check_rows(emulate_device(xe, w1, w2, act), R, "emulated")
    assert 1e-3 < err < 3e-2            # the roundings are there, and the bound is not vacuous


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_planted_row_mistakes_fail(act):
    xe, w1, w2 = make(act, 96, 256, 512, 2)
    R = ExpertRows(xe, w1, w2, act)
    # a K block of 16 hidden columns left out of the down projection
    with pytest.raises(AssertionError):
        check_rows(emulate_device(xe, w1, w2, act, drop_k=slice(128, 144)), R, "dropped K block")
    good = emulate_device(xe, w1, w2, act)
    # two rows swapped (a wrong slot)
    bad = good.copy()
    bad[[3, 4]] = bad[[4, 3]]
    with pytest.raises(AssertionError):
        check_rows(bad, R, "swapped rows")
    # every output 5% too large (a wrong scale in the epilogue)
    with pytest.raises(AssertionError):
        check_rows(f32_to_bf16_bits(bits_to_f32(good) * np.float32(1.05)), R, "scaled")


def _branch_case(seed, act="swiglu", n_tok=40, k=3, n_exp=4, d=128, f=256):
    """Tokens each summing k of n_exp experts with gates; returns the
    device-emulated branch, its BranchBound, and the pieces."""
    rng = np.random.default_rng(seed)
    experts = [make(act, n_tok, d, f, 100 * seed + e)[1:] for e in range(n_exp)]
    xe = f32_to_bf16_bits(rng.standard_normal((n_tok, d), dtype=np.float32))
    choice = np.array([rng.choice(n_exp, size=k, replace=False) for _ in range(n_tok)])
    gate = rng.uniform(0.05, 1.0, size=(n_tok, k)).astype(np.float32)
    rows = [ExpertRows(xe, w1, w2, act) for (w1, w2) in experts]
    ydev = [bits_to_f32(emulate_device(xe, w1, w2, act)) for (w1, w2) in experts]
    bb = BranchBound(n_tok, d)
    acc = np.zeros((n_tok, d), dtype=np.float32)
    for t in range(n_tok):
        for r in range(k):
            e = choice[t, r]
            bb.add(t, float(gate[t, r]), rows[e], t)
            acc[t] += gate[t, r] * ydev[e][t]
    return f32_to_bf16_bits(acc), bb, (choice, gate, ydev)


def test_emulated_branch_within_bound():
    got, bb, _ = _branch_case(3)
    err, floor, worst = check_branch(got, bb)
    assert err < 3e-2 and floor > 0 and worst > err


def test_planted_branch_mistakes_fail():
    got, bb, (choice, gate, ydev) = _branch_case(4)
    # one token loses its last expert's contribution (a dropped list entry)
    bad = bits_to_f32(got).copy()
    bad[7] -= gate[7, -1] * ydev[choice[7, -1]][7]
    with pytest.raises(AssertionError):
        check_branch(f32_to_bf16_bits(bad), bb)
    # two tokens' rows exchanged
    bad = got.copy()
    bad[[1, 2]] = bad[[2, 1]]
    with pytest.raises(AssertionError):
        check_branch(bad, bb)
    # the residual is expected but missing
    res = bits_to_f32(f32_to_bf16_bits(np.ones_like(bb.branch, dtype=np.float32))).astype(np.float64)
    with pytest.raises(AssertionError):
        check_branch(got, bb, res)
