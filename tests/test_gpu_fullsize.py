"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Router logits, selection, routing map, drops and dispatch
are compared in full (bit-exact given the device logits); expert outputs and
layer outputs on sampled tokens, which the oracle evaluates one expert at a
time."""
import numpy as np
import pytest
import torch

from sparse_expert_dispatch_amd import workloads as W

pytestmark = pytest.mark.gpu

SAMPLES = {2: 64, 3: 48, 4: 32, 5: 16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from sparse_expert_dispatch_amd import _native
    _native.lib()


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_full_size(cid):
    from harness import compare_all, log, run_gpu
    import time
    cfg = W.FULL_CONFIGS[cid]
    t0 = time.time()
    log(f"[full] {cfg.name}: generating inputs")
    inp = W.gen_inputs(cfg)
    log(f"[full] {cfg.name}: inputs ready ({time.time() - t0:.1f}s); running on the GPU")
    g = run_gpu(cfg, inp)
    log(f"[full] {cfg.name}: GPU done ({time.time() - t0:.1f}s); comparing")
    if cid == 1:
        compare_all(cfg, inp, g)
    else:
        rng = np.random.default_rng(cid)
        tokens = np.sort(rng.choice(cfg.n, size=SAMPLES[cid], replace=False))
        compare_all(cfg, inp, g, full_ffn=False, sample_tokens=tokens)
    log(f"[full] {cfg.name}: parity ok ({time.time() - t0:.1f}s)")
    del g
    torch.cuda.empty_cache()
