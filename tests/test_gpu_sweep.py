"""Seeded sweep of small layer configurations against the oracle.

Each case is drawn from a fixed generator (numpy, seed 2024 + i) over the
options the routing configuration accepts: token or expert choice; E from 2
to 256; n from 1 to 600; k up to 8; softmax, sigmoid or sqrtsoftplus scores;
dropless or a capacity of 0.5-2x the mean load, in token or rank order;
group-limited selection; a selection bias; a Zipf logit offset; noisy
logits; normalised or raw gates; a shared expert; GELU or SwiGLU; bf16
(d, f multiples of 64) or fp32.  The forward is compared stage by stage
(logits, selection bit for bit, the map, dispatch, expert rows within their
rounding bound, the combine, the statistics) by the same checks as the
fixed-shape parity tests."""
import pytest

from sparse_expert_dispatch_amd import workloads as W
from sweep_cases import sweep_case

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case(i):
    from harness import compare_all, log, run_gpu
    cfg = sweep_case(i)
    log(f"[sweep] {cfg}")
    inp = W.gen_inputs(cfg)
    g = run_gpu(cfg, inp)
    compare_all(cfg, inp, g)
