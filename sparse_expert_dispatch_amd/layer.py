"""MoELayer: the layer forward as a sequence of the library's calls.

Allocation and sequencing only.  Every step (router, selection, routing
map, dispatch, expert FFNs, combine, statistics) is one call into
libmoe_dispatch.so on the current stream; no arithmetic happens here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _native as N


def _bytes(n: int, device) -> torch.Tensor:
    # float64 storage keeps workspaces 256-byte aligned and non-empty
    return torch.empty(max(1, (int(n) + 7) // 8), dtype=torch.float64, device=device)


class MoELayer:
    """One MoE layer with device-resident weights.

    `cfg` carries the layer's shape and routing options (the fields of
    sparse_expert_dispatch_amd.workloads.MoEConfig); `weights` holds device
    tensors wg [d,E], w1 [E, f|2f, d], w2 [E, d, f] and optionally
    logit_offset [E], sel_bias [E], noise [n,E] (standard normals of noisy
    top-k, scaled by cfg.noise_std), shared_w1, shared_w2.  bf16 tensors may
    be torch.bfloat16 or raw uint16 bit patterns.

    packed (bf16 only; default on): the expert weights are copied once, at
    construction, into the packed operand order of moe_pack_expert_weights
    and the FFNs run moe_expert_ffn_packed (same results, contiguous weight
    reads).  Later changes to weights["w1"] etc. are not seen."""

    def __init__(self, cfg, weights: dict, device="cuda", packed: Optional[bool] = None):
        self.cfg = cfg
        self.device = torch.device(device)
        self.w = weights
        n, d, E = cfg.n, cfg.d, cfg.E
        tc = cfg.direction == "tc"
        self.k = cfg.k if tc else N.moe_ec_k(n, cfg.c, E)
        cap = -1
        if tc and cfg.capacity_factor is not None:
            cap = N.moe_tc_capacity(n, self.k, E, cfg.capacity_factor)
        self.capacity = cap
        score = {"softmax": N.MOE_SOFTMAX, "sigmoid": N.MOE_SIGMOID,
                 "sqrtsoftplus": N.MOE_SQRTSOFTPLUS}[cfg.score]
        order = {"token": N.MOE_TOKEN_MAJOR,
                 "rank": N.MOE_RANK_MAJOR}[getattr(cfg, "capacity_order", "token")]
        self.rcfg = N.make_cfg(n, d, E, self.k,
                               N.MOE_TOKEN_CHOICE if tc else N.MOE_EXPERT_CHOICE, score,
                               cfg.n_group, cfg.topk_group, cfg.group_topm, int(cfg.norm_topk), cap,
                               order if tc else N.MOE_TOKEN_MAJOR)
        self.noise_std = float(getattr(cfg, "noise_std", 0.0))
        self.dtype_code = N.MOE_BF16 if cfg.dtype == "bf16" else N.MOE_F32
        self.act = N.MOE_SWIGLU if cfg.act == "swiglu" else N.MOE_GELU
        edt = torch.bfloat16 if self.dtype_code == N.MOE_BF16 else torch.float32
        dev = self.device
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.M_max = N.moe_max_slots(self.rcfg)
        self.logits = torch.empty((n, E), **f32)
        self.scores_t = torch.empty((E, n), **f32) if not tc else None
        sel_shape = (n, self.k) if tc else (E, self.k)
        self.sel_idx = N.alloc(sel_shape, torch.int32, dev)
        self.sel_gate = N.alloc(sel_shape, torch.float32, dev)
        self.map = N.RouteMap(self.rcfg, dev)
        self.x_perm = N.alloc((self.M_max, d), edt, dev)
        self.y_perm = N.alloc((self.M_max, d), edt, dev)
        self.out = torch.empty((n, d), dtype=edt, device=dev)
        self.stats = torch.empty(N.MOE_NSTATS, **f32)
        self.hist = torch.empty(E + 1, **i32)
        self.ws_router = _bytes(N.moe_router_workspace_size(self.rcfg, self.dtype_code), dev)
        self.ws_route = _bytes(N.moe_route_workspace_size(self.rcfg), dev)
        self.ws_ffn = _bytes(N.moe_ffn_workspace_size(self.M_max, E, d, cfg.f, self.act,
                                                      self.dtype_code), dev)
        self.shared = bool(getattr(cfg, "shared_f", 0))
        bf16 = self.dtype_code == N.MOE_BF16
        self.packed = bf16 if packed is None else bool(packed)
        if self.packed:
            if not bf16:
                raise ValueError("packed expert weights are bf16 only")
            self.w1p, self.w2p = N.pack_ffn_weights(weights["w1"], weights["w2"], self.act)
            # the routed experts' hidden activation H [M_max, f] (bf16), in
            # the FFN workspace
            self.h = self.ws_ffn.view(torch.bfloat16)[:self.M_max * cfg.f].view(self.M_max, cfg.f)
            self.ws_gemm = _bytes(N.MOE_GEMM_WS_BYTES, dev)     # the split GEMM calls' tile counters
            if self.shared:
                self.shared_w1p, self.shared_w2p = N.pack_ffn_weights(weights["shared_w1"],
                                                                      weights["shared_w2"], self.act)
        if self.shared:
            self.shared_out = torch.empty((n, d), dtype=edt, device=dev)
            self.shared_offsets = torch.tensor([0, n], **i32)
            self.ws_shared = _bytes(N.moe_ffn_workspace_size(n, 1, d, cfg.shared_f, self.act,
                                                             self.dtype_code), dev)

    # The stages, in order; each is one library call.
    def route(self, x, stream=None):
        w = self.w
        tc = self.rcfg.dir == N.MOE_TOKEN_CHOICE
        noise = w.get("noise") if self.noise_std else None
        N.moe_router(x, w["wg"], w.get("logit_offset"), self.rcfg, self.logits, None,
                     None if tc else self.scores_t, self.ws_router, stream, noise, self.noise_std)
        N.moe_select(self.logits, None if tc else self.scores_t, w.get("sel_bias"), self.rcfg,
                     self.sel_idx, self.sel_gate, self.ws_route, stream)
        N.moe_build_map(self.sel_idx, self.sel_gate, self.rcfg, self.map, self.ws_route, stream)

    def dispatch(self, x, stream=None):
        """X_perm = P X as its own gather (the packed FFN fuses it instead)."""
        N.moe_dispatch(x, self.map, self.x_perm, stream)

    def experts(self, x, stream=None):
        if not self.packed:
            self.dispatch(x, stream)
        self.expert_ffn(x, stream)

    def routed_up(self, x, stream=None):
        """Packed weights: the routed experts' up projection + activation into
        H, its rows gathered from x through the map's slot_token (the
        dispatch fused in)."""
        N.moe_expert_up_packed(x, self.map.expert_offset, self.w1p, self.act, self.h, self.ws_gemm, stream,
                               row_index=self.map.slot_token, m_max=self.M_max)

    def routed_down(self, stream=None):
        """Packed weights: the routed experts' down projection, H -> Y_perm."""
        N.moe_expert_down_packed(self.h, self.map.expert_offset, self.w2p, self.y_perm, self.ws_gemm, stream)

    def shared_expert(self, x, stream=None):
        """The always-on shared expert on every token (packed weights)."""
        N.moe_expert_ffn_packed(x, self.shared_offsets, self.shared_w1p, self.shared_w2p, self.act,
                                self.shared_out, self.ws_shared, stream)

    def expert_ffn(self, x, stream=None):
        """The routed experts (and the shared expert on x).  Packed weights:
        the up GEMM gathers its rows from x through the map's slot_token
        (dispatch fused in); otherwise it reads the dispatched X_perm."""
        w = self.w
        if self.packed:
            self.routed_up(x, stream)
            self.routed_down(stream)
            if self.shared:
                self.shared_expert(x, stream)
            return
        N.moe_expert_ffn(self.x_perm, self.map.expert_offset, w["w1"], w["w2"], self.act,
                         self.y_perm, self.ws_ffn, stream)
        if self.shared:
            N.moe_expert_ffn(x, self.shared_offsets, w["shared_w1"], w["shared_w2"], self.act,
                             self.shared_out, self.ws_shared, stream)

    def combine(self, x, residual: bool = True, stream=None):
        N.moe_combine(self.y_perm, self.map, self.cfg.n, x if residual else None,
                      self.shared_out if self.shared else None, self.out, stream)

    def balance_stats(self, stream=None):
        N.moe_balance_stats(self.logits, self.map, self.rcfg, self.cfg.lb_coef, self.cfg.z_coef,
                            self.stats, self.hist, self.ws_route, stream)

    def update_bias(self, gamma: float, stream=None):
        """Loss-free balancing step on weights["sel_bias"] from this step's
        per-expert loads (after route())."""
        N.moe_update_bias(self.map.expert_count, self.rcfg, gamma, self.w["sel_bias"], stream)

    def forward(self, x: torch.Tensor, residual: bool = True, stats: bool = True,
                stream=None) -> torch.Tensor:
        """out = residual + shared expert + gate-weighted routed experts.
        Results (and every intermediate) stay in this object's buffers."""
        self.route(x, stream)
        self.experts(x, stream)
        self.combine(x, residual, stream)
        if stats:
            self.balance_stats(stream)
        return self.out


    def backward(self, x: torch.Tensor, dout: torch.Tensor, residual: bool = True, stream=None) -> dict:
        """Gradients of <dout, out> + lb_loss + z_loss for the last forward(x)
        (routing fixed; the coefficients are the config's lb_coef, z_coef).
        Returns device tensors: dx [n, d] (dtype), dwg [d, E], d_offset [E],
        dw1 / dw2 (fp32, the natural weight shapes) and, with a shared expert,
        shared_dw1 / shared_dw2; plus the intermediates dz, d_gate, dx_perm.
        On packed weights the forward never materialised X_perm; this runs
        the standalone dispatch for it first."""
        cfg, w = self.cfg, self.w
        n, d, E = cfg.n, cfg.d, cfg.E
        if not hasattr(self, "bw"):
            dev = self.device
            edt = self.out.dtype
            f32 = dict(dtype=torch.float32, device=dev)
            bw = dict(dy_perm=N.alloc((self.M_max, d), edt, dev), d_gate=N.alloc((self.M_max,), torch.float32, dev),
                      dx_perm=N.alloc((self.M_max, d), edt, dev), dw1=torch.empty(w["w1"].shape, **f32),
                      dw2=torch.empty(w["w2"].shape, **f32), dz=torch.empty((n, E), **f32),
                      dx_r=torch.empty((n, d), dtype=edt, device=dev), dx=torch.empty((n, d), dtype=edt, device=dev),
                      dwg=torch.empty((d, E), **f32), d_offset=torch.empty(E, **f32))
            sizes = [N.moe_ffn_backward_workspace_size(self.M_max, E, d, cfg.f, self.act, self.dtype_code),
                     N.moe_router_backward_workspace_size(self.rcfg, self.dtype_code)]
            if self.shared:
                bw["dx_shared"] = torch.empty((n, d), dtype=edt, device=dev)
                bw["shared_dw1"] = torch.empty(w["shared_w1"].shape, **f32)
                bw["shared_dw2"] = torch.empty(w["shared_w2"].shape, **f32)
                sizes.append(N.moe_ffn_backward_workspace_size(n, 1, d, cfg.shared_f, self.act, self.dtype_code))
            bw["ws"] = _bytes(max(sizes), dev)
            self.bw = bw
        b = self.bw
        if self.packed:
            self.dispatch(x, stream)
        N.moe_combine_backward(dout, self.y_perm, self.map, b["dy_perm"], b["d_gate"], stream)
        N.moe_expert_ffn_backward(self.x_perm, self.map.expert_offset, w["w1"], w["w2"], self.act, b["dy_perm"],
                                  b["dx_perm"], b["dw1"], b["dw2"], b["ws"], stream)
        if self.shared:
            N.moe_expert_ffn_backward(x, self.shared_offsets, w["shared_w1"], w["shared_w2"], self.act, dout,
                                      b["dx_shared"], b["shared_dw1"], b["shared_dw2"], b["ws"], stream)
        N.moe_gate_backward(self.logits, self.sel_idx, b["d_gate"], self.rcfg, self.map, cfg.lb_coef, cfg.z_coef,
                            b["dz"], stream)
        N.moe_router_backward(x, w["wg"], b["dz"], self.rcfg, dout if residual else None, b["dx_r"], b["dwg"],
                              b["d_offset"], b["ws"], stream)
        N.moe_dispatch_backward(b["dx_perm"], self.map, n, b["dx_r"], b.get("dx_shared"), b["dx"], stream)
        out = {key: b[key] for key in ("dx", "dwg", "d_offset", "dw1", "dw2", "dz", "d_gate", "dx_perm", "dy_perm")}
        if self.shared:
            out["shared_dw1"], out["shared_dw2"] = b["shared_dw1"], b["shared_dw2"]
        return out

    def capture(self, x: torch.Tensor, residual: bool = True, stats: bool = True):
        """Record one forward into a HIP graph (torch.cuda.CUDAGraph) and
        return it; graph.replay() recomputes every buffer of this layer from
        the current contents of `x` (a fixed device buffer) with one launch.
        An eager forward runs first, so the library's one-time host queries
        (occupancy, LDS attributes) stay outside the capture.  Every stage is
        a kernel launch on the current stream: no memsets, no host
        synchronisation, no allocation."""
        self.forward(x, residual, stats)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x, residual, stats)
        return graph

    def capture_step(self, x: torch.Tensor, dout: torch.Tensor, residual: bool = True):
        """Record one forward and its backward (one training step of the
        layer) into a HIP graph; replays recompute every output and gradient
        buffer from the current contents of `x` and `dout`.  An eager step
        runs first, so the gradient buffers are allocated and the library's
        one-time host queries happen outside the capture."""
        self.forward(x, residual)
        self.backward(x, dout, residual)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x, residual)
            self.backward(x, dout, residual)
        return graph


def to_device(a, device="cuda") -> Optional[torch.Tensor]:
    """numpy array (float32, int32, or bf16 as uint16) -> device tensor
    (bf16 bit patterns become torch.bfloat16 without any conversion)."""
    import numpy as np
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)
