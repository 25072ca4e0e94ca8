"""Seeded small layer configurations for the sweep tests (inputs only: no
arithmetic of the method).  Case i is drawn from numpy's generator with
seed 2024 + i over the options the routing configuration accepts; see
test_gpu_sweep.py for the list."""
import numpy as np

from sparse_expert_dispatch_amd import workloads as W


def sweep_case(i: int) -> W.MoEConfig:
    rng = np.random.default_rng(2024 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    bf16 = rng.random() < 0.75
    E = int(pick([2, 3, 5, 8, 16, 24, 40, 64, 96, 128, 160, 256]))
    n = int(rng.integers(1, 601))
    if bf16:
        d, f = int(pick([64, 128, 192, 256])), int(pick([64, 128, 192]))
    else:
        d, f = int(pick([48, 64, 96, 130])), int(pick([32, 64, 100]))
    kw = dict(name=f"sweep{i}", cfg_id=100 + i, n=n, d=d, E=E, f=f, act=str(pick(["gelu", "swiglu"])),
              dtype="bf16" if bf16 else "f32", seed=int(rng.integers(1 << 30)),
              norm_topk=bool(rng.random() < 0.7))
    if rng.random() < 0.25:
        # k = n c / E tokens per expert must not exceed n: c <= E
        kw.update(direction="ec", score="softmax", c=min(float(pick([0.5, 1.0, 2.0, 4.0])), float(E)),
                  norm_topk=True)
    else:
        k = int(rng.integers(1, min(8, E) + 1))
        kw.update(direction="tc", k=k, score=str(pick(["softmax", "sigmoid", "sqrtsoftplus"])),
                  capacity_factor=pick([None, None, 0.5, 1.25, 2.0]),
                  capacity_order=str(pick(["token", "token", "rank"])))
        if E % 4 == 0 and rng.random() < 0.35 and k <= 2 * (E // 4):
            kw.update(n_group=4, topk_group=2, group_topm=int(min(pick([1, 2]), E // 4)))
        if kw["score"] != "softmax" and rng.random() < 0.5:
            kw.update(bias_halfwidth=0.05)
        if rng.random() < 0.2:
            kw.update(noise_std=0.5)
    if rng.random() < 0.3:
        kw.update(zipf_offset_s=1.1)
    if rng.random() < 0.25:
        kw.update(shared_f=int(pick([64, 128])) if bf16 else 32)
    return W.MoEConfig(**kw)
