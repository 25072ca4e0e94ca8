"""The layer forward (and a forward + backward step) captured in a HIP
graph: every replay, with the program's own eager work and
synchronisations between replays, must give the eager result bit for bit
(outputs, routing map, statistics, gradients)."""
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


@pytest.mark.parametrize("cid", [2, 3])
def test_graph_training_step_matches_eager(cid):
    """Forward + backward in one graph (expert choice GELU; top-8 SwiGLU):
    outputs and every gradient bit for bit against eager steps."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from harness import host, log, upload
    from sparse_expert_dispatch_amd.layer import MoELayer, to_device
    cfg = W.SMALL_CONFIGS[cid]
    inp = W.gen_inputs(cfg)
    w = upload(cfg, inp)
    rng = np.random.default_rng(60 + cid)
    xs = [to_device(inp["x"])] + [to_device(W.f32_to_bf16_bits(rng.standard_normal(inp["x"].shape, dtype=np.float32)))
                                  for _ in range(2)]
    douts = [to_device(W.f32_to_bf16_bits(rng.standard_normal(inp["x"].shape, dtype=np.float32))) for _ in xs]
    x_static, d_static = xs[0].clone(), douts[0].clone()
    graphed = MoELayer(cfg, w)
    graph = graphed.capture_step(x_static, d_static)
    eager = MoELayer(cfg, w)
    for rep in range(2):
        for i, (xi, di) in enumerate(zip(xs, douts)):
            x_static.copy_(xi)
            d_static.copy_(di)
            scratch = (di.float() * 3).sum()          # unrelated eager work between replays
            graph.replay()
            torch.cuda.synchronize()
            eager.forward(xi)
            ge = eager.backward(xi, di)
            torch.cuda.synchronize()
            assert np.array_equal(host(graphed.out).view(np.uint8), host(eager.out).view(np.uint8)), (rep, i, "out")
            for key in ("dx", "dwg", "d_offset", "dw1", "dw2", "dz"):
                a, b = host(graphed.bw[key]), host(ge[key])
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, i, key)
            assert torch.isfinite(scratch)
    log(f"  {cfg.name}: {2 * len(xs)} graph replays of forward + backward equal the eager step")
