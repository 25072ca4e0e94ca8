"""Seeded synthetic workloads for the MoE-layer forward.

This module only *creates inputs*: configuration shapes and seeded random
tensors.  It holds none of the layer's arithmetic (no capacity, no k, no
scores), so both the HIP path and the CPU oracle can consume its output
without sharing any of the method.

Shapes and distributions follow the five workloads of the MoE-routing pages
(token choice vs expert choice; sigmoid gating with selection bias and
group-limited routing; shared plus routed experts).  Where a distribution is
not stated it is read as: X ~ N(0,1), W_g ~ N(0, 1/d), expert weights
~ N(0, 1/fan_in) (fan_in = d for the up projection, f for the down
projection).

Every tensor has its own random stream, ``SeedSequence([seed, cfg_id,
tensor_id, expert])``, so expert weights can be regenerated one expert at a
time (the oracle never needs all of a 22 GB weight set at once).

bf16 tensors are returned as ``uint16`` bit patterns, rounded from float32
normals with round-to-nearest-even; fp32 tensors as ``float32``.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# tensor ids for the per-tensor seed streams
_T_X, _T_WG, _T_W1, _T_W2, _T_OFFSET, _T_BIAS, _T_SW1, _T_SW2, _T_NOISE = range(9)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One MoE-layer workload.

    direction: "tc" (token choice, ``k`` experts per token) or "ec" (expert
    choice, capacity factor ``c``; tokens per expert is derived by the
    library).  ``capacity_factor`` None means dropless token choice.
    """
    name: str
    cfg_id: int
    n: int
    d: int
    E: int
    f: int
    act: str                       # "gelu" | "swiglu"
    dtype: str                     # "f32" | "bf16"
    direction: str = "tc"          # "tc" | "ec"
    score: str = "softmax"         # "softmax" | "sigmoid" | "sqrtsoftplus"
    k: int = 1                     # token choice: experts per token
    c: float = 0.0                 # expert choice: capacity factor
    capacity_factor: Optional[float] = None   # token choice; None = dropless
    norm_topk: bool = True         # renormalise gates over the selected experts
    n_group: int = 1
    topk_group: int = 1
    group_topm: int = 1            # group score = sum of the top-m keys of the group
    wg_var_scale: float = 1.0      # W_g ~ N(0, wg_var_scale / d)
    zipf_offset_s: Optional[float] = None     # per-expert additive logit offset
    bias_halfwidth: Optional[float] = None    # selection bias ~ U(-h, h)
    shared_f: int = 0              # always-on shared expert hidden size (0 = none)
    capacity_order: str = "token"  # capacity priority: "token" (token-major) | "rank" (rank-major)
    noise_std: float = 0.0         # noisy top-k: logits += noise_std * N(0, 1) per (token, expert)
    lb_coef: float = 0.01
    z_coef: float = 0.001
    seed: int = 0

    @property
    def w1_rows(self) -> int:
        return 2 * self.f if self.act == "swiglu" else self.f

    def scaled(self, name: str, **kw) -> "MoEConfig":
        return dataclasses.replace(self, name=name, **kw)


# The five workloads of the pages, at full size.
C1 = MoEConfig("tc_top2_fp32_n256", 1, n=256, d=64, E=8, f=128, act="gelu", dtype="f32",
               direction="tc", score="softmax", k=2, capacity_factor=1.25, norm_topk=True)
C2 = MoEConfig("ec_c2_bf16_n4096_d2048_e64", 2, n=4096, d=2048, E=64, f=4096, act="gelu",
               dtype="bf16", direction="ec", score="softmax", c=2.0)
C3 = MoEConfig("tc_top8_dropless_zipf_bf16_n8192_d2048_e64", 3, n=8192, d=2048, E=64, f=1024,
               act="swiglu", dtype="bf16", direction="tc", score="softmax", k=8,
               capacity_factor=None, norm_topk=True, zipf_offset_s=1.1)
C4 = MoEConfig("switch_top1_cap160_bf16_n16384_d4096_e128", 4, n=16384, d=4096, E=128, f=8192,
               act="gelu", dtype="bf16", direction="tc", score="softmax", k=1,
               capacity_factor=1.25, norm_topk=False, wg_var_scale=2.0)
C5 = MoEConfig("sigmoid_bias_group_shared_bf16_n4096_d7168_e256", 5, n=4096, d=7168, E=256,
               f=2048, act="swiglu", dtype="bf16", direction="tc", score="sigmoid", k=8,
               capacity_factor=None, norm_topk=True, n_group=8, topk_group=4, group_topm=1,
               bias_halfwidth=0.1, shared_f=2048)

FULL_CONFIGS = {c.cfg_id: c for c in (C1, C2, C3, C4, C5)}

# A decode step of an OLMoE-shaped layer: 64 tokens, top-8 of 64 SwiGLU
# experts, dropless.  Each expert sees about 8 rows, so the grouped GEMM is
# weight streaming with almost no arithmetic per byte.
DECODE = MoEConfig("decode_top8_swiglu_bf16_n64_d2048_e64", 6, n=64, d=2048, E=64, f=1024,
                   act="swiglu", dtype="bf16", direction="tc", score="softmax", k=8,
                   capacity_factor=None, norm_topk=True)
EXTRA_CONFIGS = {"decode": DECODE}

# Reduced shapes of the same five workloads: small enough for the oracle to
# finish in seconds, large enough to span several GEMM tiles and leave ragged
# per-expert tails.
SMALL_CONFIGS = {
    1: C1,
    2: C2.scaled("ec_c2_bf16_small", n=1000, d=256, E=16, f=512),
    3: C3.scaled("tc_top8_dropless_zipf_bf16_small", n=1536, d=256, E=16, f=192),
    4: C4.scaled("switch_top1_cap_bf16_small", n=2000, d=384, E=16, f=640),
    5: C5.scaled("sigmoid_bias_group_shared_bf16_small", n=700, d=512, E=64, f=128,
                 n_group=8, topk_group=4, shared_f=256),
}


def _rng(cfg: MoEConfig, tensor_id: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([cfg.seed, cfg.cfg_id, tensor_id, expert])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal(cfg: MoEConfig, tensor_id: int, expert: int, shape, std: float) -> np.ndarray:
    g = _rng(cfg, tensor_id, expert)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a) if cfg.dtype == "bf16" else a


def gen_x(cfg: MoEConfig) -> np.ndarray:
    return _normal(cfg, _T_X, 0, (cfg.n, cfg.d), 1.0)


def gen_wg(cfg: MoEConfig) -> np.ndarray:
    """Router weight in the pages' [d, E] layout."""
    return _normal(cfg, _T_WG, 0, (cfg.d, cfg.E), math.sqrt(cfg.wg_var_scale / cfg.d))


def gen_w1_expert(cfg: MoEConfig, e: int) -> np.ndarray:
    """Up projection of expert e, [f, d] (SwiGLU: [2f, d], gate rows first)."""
    return _normal(cfg, _T_W1, e, (cfg.w1_rows, cfg.d), math.sqrt(1.0 / cfg.d))


def gen_w2_expert(cfg: MoEConfig, e: int) -> np.ndarray:
    """Down projection of expert e, [d, f]."""
    return _normal(cfg, _T_W2, e, (cfg.d, cfg.f), math.sqrt(1.0 / cfg.f))


def gen_shared_w1(cfg: MoEConfig) -> np.ndarray:
    rows = 2 * cfg.shared_f if cfg.act == "swiglu" else cfg.shared_f
    return _normal(cfg, _T_SW1, 0, (rows, cfg.d), math.sqrt(1.0 / cfg.d))


def gen_shared_w2(cfg: MoEConfig) -> np.ndarray:
    return _normal(cfg, _T_SW2, 0, (cfg.d, cfg.shared_f), math.sqrt(1.0 / cfg.shared_f))


def gen_logit_offset(cfg: MoEConfig) -> Optional[np.ndarray]:
    """Zipf-shaped per-expert logit offset: -s*ln(rank+1) over a random rank
    permutation, so that softmax preferences fall off as (rank+1)^-s."""
    if cfg.zipf_offset_s is None:
        return None
    rank = _rng(cfg, _T_OFFSET).permutation(cfg.E)
    return (-cfg.zipf_offset_s * np.log(rank + 1.0)).astype(np.float32)


def gen_sel_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    if cfg.bias_halfwidth is None:
        return None
    h = cfg.bias_halfwidth
    return _rng(cfg, _T_BIAS).uniform(-h, h, size=cfg.E).astype(np.float32)


def gen_noise(cfg: MoEConfig) -> Optional[np.ndarray]:
    """Standard normals [n, E] for noisy top-k (scaled by noise_std inside
    the router); the method's random numbers are inputs, drawn here."""
    if not cfg.noise_std:
        return None
    return _rng(cfg, _T_NOISE).standard_normal((cfg.n, cfg.E), dtype=np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gen_expert_weights(cfg: MoEConfig, experts=None, threads: Optional[int] = None):
    """Stacked W1 [E', w1_rows, d] and W2 [E', d, f] for the given experts
    (default: all), generated in parallel one expert per task."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    w1 = np.empty((len(experts), cfg.w1_rows, cfg.d), dtype=dt)
    w2 = np.empty((len(experts), cfg.d, cfg.f), dtype=dt)

    def job(i):
        e = experts[i]
        w1[i] = gen_w1_expert(cfg, e)
        w2[i] = gen_w2_expert(cfg, e)

    with ThreadPoolExecutor(max_workers=threads or _threads()) as ex:
        list(ex.map(job, range(len(experts))))
    return w1, w2


def gen_inputs(cfg: MoEConfig, with_experts: bool = True, threads: Optional[int] = None) -> dict:
    """All inputs of one layer forward as numpy arrays (see module doc)."""
    out = {
        "x": gen_x(cfg),
        "wg": gen_wg(cfg),
        "logit_offset": gen_logit_offset(cfg),
        "sel_bias": gen_sel_bias(cfg),
        "noise": gen_noise(cfg),
    }
    if with_experts:
        out["w1"], out["w2"] = gen_expert_weights(cfg, threads=threads)
    if cfg.shared_f:
        out["shared_w1"] = gen_shared_w1(cfg)
        out["shared_w2"] = gen_shared_w2(cfg)
    return out
