"""The layer forward captured in a HIP graph: every replay, with the
program's own eager work and synchronisations between replays, must give
the eager result bit for bit (outputs, routing map and statistics)."""
import numpy as np
import pytest
import torch

from sparse_expert_dispatch_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_graph_replays_match_eager(cid):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from harness import host, log, upload
    from sparse_expert_dispatch_amd.layer import MoELayer, to_device
    cfg = W.SMALL_CONFIGS[cid]
    inp = W.gen_inputs(cfg)
    w = upload(cfg, inp)
    xs = [to_device(inp["x"])]
    rng = np.random.default_rng(40 + cid)
    for _ in range(3):      # other token batches of the same shape (bf16 bit patterns)
        xs.append(to_device(W.f32_to_bf16_bits(rng.standard_normal(inp["x"].shape, dtype=np.float32))))
    x_static = xs[0].clone()
    graphed = MoELayer(cfg, w)
    graph = graphed.capture(x_static)
    eager = MoELayer(cfg, w)
    keys = ("out", "logits", "sel_idx", "sel_gate", "stats", "hist")
    for rep in range(2):
        for i, xi in enumerate(xs):
            x_static.copy_(xi)
            scratch = (xi.float() * 2).sum()          # unrelated eager work between replays
            graph.replay()
            torch.cuda.synchronize()
            eager.forward(xi)
            torch.cuda.synchronize()
            for key in keys:
                a, b = host(getattr(graphed, key)), host(getattr(eager, key))
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, i, key)
            for f in ("expert_offset", "slot_token", "token_slot"):
                assert np.array_equal(host(getattr(graphed.map, f)), host(getattr(eager.map, f))), (rep, i, f)
            assert torch.isfinite(scratch)
    log(f"  {cfg.name}: {2 * len(xs)} graph replays equal the eager forward")
