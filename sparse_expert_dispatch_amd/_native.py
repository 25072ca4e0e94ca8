"""ctypes binding of libmoe_dispatch.so (the C ABI in include/moe_dispatch.h).

Argument marshalling only: every function here checks tensor placement,
dtype and contiguity, turns tensors into raw device pointers and calls the
library, which does all the work in its HIP kernels.  PyTorch supplies device
memory and the current stream.  There is no fallback: if the library is not
built, or a call fails, an exception says so.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmoe_dispatch.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID, MOE_SQRTSOFTPLUS = 0, 1, 2
MOE_TOKEN_MAJOR, MOE_RANK_MAJOR = 0, 1
MOE_TOKEN_CHOICE, MOE_EXPERT_CHOICE = 0, 1
MOE_GELU, MOE_SWIGLU = 0, 1
MOE_NSTATS = 8
MOE_GEMM_WS_BYTES = 256
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
STAT_NAMES = ("lb_loss", "z_loss", "max_vio", "max_load_share", "n_kept", "n_dropped",
              "tokens_without_expert", "max_experts_per_token")

EXPORTED = ("moe_ec_k", "moe_tc_capacity", "moe_max_slots", "moe_token_list_len",
            "moe_router_workspace_size",
            "moe_route_workspace_size", "moe_ffn_workspace_size", "moe_router", "moe_select",
            "moe_build_map", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_balance_stats",
            "moe_update_bias", "moe_pack_expert_weights", "moe_expert_ffn_packed",
            "moe_expert_up_packed", "moe_expert_down_packed", "moe_expert_ffn_packed_noalloc",
            "moe_combine_backward", "moe_ffn_backward_workspace_size", "moe_expert_ffn_backward",
            "moe_gate_backward", "moe_router_backward_workspace_size", "moe_router_backward",
            "moe_dispatch_backward", "moe_status_string", "moe_last_error")


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class RouteCfg(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("n", "d", "E", "k", "dir", "score", "n_group", "topk_group", "group_topm",
                 "norm_topk", "capacity", "capacity_order")]


class RouteMapC(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("expert_count", "expert_offset", "slot_token", "slot_gate", "assign_slot",
                 "token_offset", "token_slot", "n_kept")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_expert_dispatch_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32, F64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                 ctypes.c_float, ctypes.c_double)
    CFG = ctypes.POINTER(RouteCfg)
    MAP = ctypes.POINTER(RouteMapC)
    SZP = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "moe_ec_k": (I32, [I32, F64, I32]),
        "moe_tc_capacity": (I32, [I32, I32, I32, F64]),
        "moe_max_slots": (I64, [CFG]),
        "moe_token_list_len": (I64, [CFG]),
        "moe_router_workspace_size": (I32, [CFG, I32, SZP]),
        "moe_route_workspace_size": (I32, [CFG, SZP]),
        "moe_ffn_workspace_size": (I32, [I64, I32, I32, I32, I32, I32, SZP]),
        "moe_router": (I32, [P, P, I32, P, P, F32, CFG, P, P, P, P, SZ, P]),
        "moe_select": (I32, [P, P, P, CFG, P, P, P, SZ, P]),
        "moe_build_map": (I32, [P, P, CFG, MAP, P, SZ, P]),
        "moe_dispatch": (I32, [P, I32, I32, I32, MAP, I64, P, P]),
        "moe_expert_ffn": (I32, [P, I32, P, I32, I32, I32, I32, P, P, I64, P, P, SZ, P]),
        "moe_combine": (I32, [P, I32, MAP, I32, I32, P, P, P, P]),
        "moe_balance_stats": (I32, [P, MAP, CFG, F32, F32, P, P, P, SZ, P]),
        "moe_update_bias": (I32, [P, CFG, F32, P, P]),
        "moe_pack_expert_weights": (I32, [P, I32, I32, I32, I32, P, P]),
        "moe_expert_ffn_packed": (I32, [P, I32, P, P, I32, I32, I32, I32, P, P, I64, P, P, SZ, P]),
        "moe_expert_up_packed": (I32, [P, I32, P, P, I32, I32, I32, I32, P, I64, P, P, SZ, P]),
        "moe_expert_down_packed": (I32, [P, P, I32, I32, I32, P, I64, P, P, SZ, P]),
        "moe_expert_ffn_packed_noalloc": (I32, [P, I32, P, P, I32, I32, I32, I32, P, P, I64, P, P]),
        "moe_combine_backward": (I32, [P, P, I32, I32, I32, MAP, I64, P, P, P]),
        "moe_ffn_backward_workspace_size": (I32, [I64, I32, I32, I32, I32, I32, SZP]),
        "moe_expert_ffn_backward": (I32, [P, I32, P, I32, I32, I32, I32, P, P, P, I64, P, P, P, P, SZ, P]),
        "moe_gate_backward": (I32, [P, P, P, CFG, MAP, F32, F32, P, P]),
        "moe_router_backward_workspace_size": (I32, [CFG, I32, SZP]),
        "moe_router_backward": (I32, [P, P, I32, P, CFG, P, P, P, P, P, SZ, P]),
        "moe_dispatch_backward": (I32, [P, I32, MAP, I32, I32, P, P, P, P]),
        "moe_status_string": (ctypes.c_char_p, [I32]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


# ---------------------------------------------------------------- marshalling helpers

def _ptr(t: Optional[torch.Tensor], name: str, dtypes=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return _addr(t)


def _addr(t: torch.Tensor) -> int:
    """Device address of t.  A zero-sized view (see alloc) reports address 0;
    pass the address of its backing storage instead, so zero-length arrays
    are never NULL at the C ABI."""
    p = t.data_ptr()
    if p == 0 and t.numel() == 0:
        p = t.untyped_storage().data_ptr() + t.storage_offset() * t.element_size()
    return p


_BF16_STORAGE = (torch.bfloat16, torch.uint16, torch.int16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype in _BF16_STORAGE:
        return MOE_BF16
    raise TypeError(f"unsupported element type {t.dtype} (float32 or bfloat16)")


def _elem_dtypes(code: int):
    return _F32 if code == MOE_F32 else _BF16_STORAGE


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        L = lib()
        raise MoEError(status, where, f"{L.moe_status_string(status).decode()}: "
                                      f"{L.moe_last_error().decode()}")


def make_cfg(n, d, E, k, direction=MOE_TOKEN_CHOICE, score=MOE_SOFTMAX, n_group=1, topk_group=1,
             group_topm=1, norm_topk=1, capacity=-1, capacity_order=MOE_TOKEN_MAJOR) -> RouteCfg:
    return RouteCfg(int(n), int(d), int(E), int(k), int(direction), int(score), int(n_group),
                    int(topk_group), int(group_topm), int(norm_topk), int(capacity),
                    int(capacity_order))


def alloc(shape, dtype, device="cuda") -> torch.Tensor:
    """torch.empty(shape) backed by at least one element: zero-sized tensors
    (expert choice with k = 0 has no slots) are views of a one-element
    buffer, whose address the marshalling passes, so the C ABI's non-NULL
    checks hold for them too."""
    numel = 1
    for s in shape:
        numel *= int(s)
    return torch.empty(max(numel, 1), dtype=dtype, device=device)[:numel].view(*shape)


class RouteMap:
    """Device buffers of a routing map (allocated with torch)."""

    FIELDS = ("expert_count", "expert_offset", "slot_token", "slot_gate", "assign_slot",
              "token_offset", "token_slot", "n_kept")

    def __init__(self, cfg: RouteCfg, device="cuda"):
        M = moe_max_slots(cfg)
        n, E, k = cfg.n, cfg.E, cfg.k
        i32 = dict(dtype=torch.int32, device=device)
        self.M_max = M
        self.expert_count = torch.empty(E, **i32)
        self.expert_offset = torch.empty(E + 1, **i32)
        self.slot_token = alloc((M,), torch.int32, device)
        self.slot_gate = alloc((M,), torch.float32, device)
        self.assign_slot = alloc((n, k) if cfg.dir == MOE_TOKEN_CHOICE else (E, k), torch.int32, device)
        self.token_offset = torch.empty(n + 1, **i32)
        self.token_slot = alloc((moe_token_list_len(cfg),), torch.int32, device)
        self.n_kept = torch.empty(1, **i32)

    def c(self) -> RouteMapC:
        return RouteMapC(*[_addr(getattr(self, f)) for f in self.FIELDS])


# ---------------------------------------------------------------- the C ABI, one to one

def moe_ec_k(n: int, c: float, E: int) -> int:
    return lib().moe_ec_k(int(n), float(c), int(E))


def moe_tc_capacity(n: int, k: int, E: int, cf: float) -> int:
    return lib().moe_tc_capacity(int(n), int(k), int(E), float(cf))


def moe_max_slots(cfg: RouteCfg) -> int:
    v = lib().moe_max_slots(ctypes.byref(cfg))
    if v < 0:
        _check(MOE_ERR_INVALID_ARG, "moe_max_slots")
    return v


def moe_token_list_len(cfg: RouteCfg) -> int:
    v = lib().moe_token_list_len(ctypes.byref(cfg))
    if v < 0:
        _check(MOE_ERR_INVALID_ARG, "moe_token_list_len")
    return v


def moe_router_workspace_size(cfg: RouteCfg, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_router_workspace_size(ctypes.byref(cfg), int(dtype), ctypes.byref(out)),
           "moe_router_workspace_size")
    return out.value


def moe_route_workspace_size(cfg: RouteCfg) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_route_workspace_size(ctypes.byref(cfg), ctypes.byref(out)),
           "moe_route_workspace_size")
    return out.value


def moe_ffn_workspace_size(M_max: int, E: int, d: int, f: int, act: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_ffn_workspace_size(int(M_max), int(E), int(d), int(f), int(act), int(dtype),
                                        ctypes.byref(out)), "moe_ffn_workspace_size")
    return out.value


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return _ptr(ws, "ws"), ws.numel() * ws.element_size()


def moe_router(x, wg, logit_offset, cfg: RouteCfg, logits, scores=None, scores_t=None, ws=None,
               stream=None, noise=None, noise_std=0.0):
    code = dtype_code(x)
    w, wb = _ws(ws)
    _check(lib().moe_router(_ptr(x, "x", _elem_dtypes(code)), _ptr(wg, "wg", _elem_dtypes(code)), code,
                            _ptr(logit_offset, "logit_offset", _F32), _ptr(noise, "noise", _F32),
                            float(noise_std), ctypes.byref(cfg),
                            _ptr(logits, "logits", _F32), _ptr(scores, "scores", _F32),
                            _ptr(scores_t, "scores_t", _F32), w, wb, _stream(stream)), "moe_router")


def moe_select(logits, scores_t, sel_bias, cfg: RouteCfg, sel_idx, sel_gate, ws=None, stream=None):
    w, wb = _ws(ws)
    _check(lib().moe_select(_ptr(logits, "logits", _F32), _ptr(scores_t, "scores_t", _F32),
                            _ptr(sel_bias, "sel_bias", _F32), ctypes.byref(cfg),
                            _ptr(sel_idx, "sel_idx", _I32), _ptr(sel_gate, "sel_gate", _F32), w, wb,
                            _stream(stream)), "moe_select")


def moe_build_map(sel_idx, sel_gate, cfg: RouteCfg, rmap: RouteMap, ws=None, stream=None):
    w, wb = _ws(ws)
    cm = rmap.c()
    _check(lib().moe_build_map(_ptr(sel_idx, "sel_idx", _I32), _ptr(sel_gate, "sel_gate", _F32),
                               ctypes.byref(cfg), ctypes.byref(cm), w, wb, _stream(stream)),
           "moe_build_map")


def moe_dispatch(x, rmap: RouteMap, x_perm, stream=None):
    code = dtype_code(x)
    n, d = x.shape
    cm = rmap.c()
    _check(lib().moe_dispatch(_ptr(x, "x", _elem_dtypes(code)), code, int(n), int(d), ctypes.byref(cm),
                              int(x_perm.shape[0]), _ptr(x_perm, "x_perm", _elem_dtypes(code)),
                              _stream(stream)), "moe_dispatch")


def moe_expert_ffn(x_perm, expert_offset, w1, w2, act: int, y_perm, ws, stream=None):
    code = dtype_code(x_perm)
    E = expert_offset.numel() - 1
    d = x_perm.shape[1]
    f = w2.shape[-1]
    w, wb = _ws(ws)
    _check(lib().moe_expert_ffn(_ptr(x_perm, "x_perm", _elem_dtypes(code)), code,
                                _ptr(expert_offset, "expert_offset", _I32), int(E), int(d), int(f),
                                int(act), _ptr(w1, "w1", _elem_dtypes(code)),
                                _ptr(w2, "w2", _elem_dtypes(code)), int(x_perm.shape[0]),
                                _ptr(y_perm, "y_perm", _elem_dtypes(code)), w, wb, _stream(stream)),
           "moe_expert_ffn")


def moe_pack_expert_weights(w, gate_up: bool, w_packed, stream=None):
    """w [E, rows, K] (or one expert's [rows, K]) bf16 -> w_packed (same shape
    and size, the packed operand order)."""
    E, rows, K = (1, *w.shape) if w.dim() == 2 else w.shape
    _check(lib().moe_pack_expert_weights(_ptr(w, "w", _elem_dtypes(MOE_BF16)), int(E), int(rows), int(K),
                                         int(bool(gate_up)), _ptr(w_packed, "w_packed", _elem_dtypes(MOE_BF16)),
                                         _stream(stream)), "moe_pack_expert_weights")


def pack_ffn_weights(w1, w2, act: int, stream=None):
    """Packed copies of one FFN's W1 [E, f or 2f, d] and W2 [E, d, f]."""
    w1p, w2p = torch.empty_like(w1), torch.empty_like(w2)
    moe_pack_expert_weights(w1, act == MOE_SWIGLU, w1p, stream)
    moe_pack_expert_weights(w2, False, w2p, stream)
    return w1p, w2p


def moe_expert_ffn_packed(x, expert_offset, w1p, w2p, act: int, y_perm, ws, stream=None, row_index=None,
                          m_max=None):
    """Packed-weight FFN.  row_index=None: x is x_perm (rows = slots).
    row_index = the map's slot_token: x is the token matrix [n, d] and the
    up GEMM gathers its rows (the dispatch fused in); m_max then gives the
    slot count (default: y_perm's rows)."""
    E = expert_offset.numel() - 1
    d = x.shape[1]
    f = w2p.shape[-1]
    M_max = int(m_max if m_max is not None else (y_perm.shape[0] if row_index is not None else x.shape[0]))
    w, wb = _ws(ws)
    bf = _elem_dtypes(MOE_BF16)
    _check(lib().moe_expert_ffn_packed(_ptr(x, "x", bf), int(x.shape[0]),
                                       _ptr(row_index, "row_index", _I32) if row_index is not None else None,
                                       _ptr(expert_offset, "expert_offset", _I32),
                                       int(E), int(d), int(f), int(act), _ptr(w1p, "w1_packed", bf),
                                       _ptr(w2p, "w2_packed", bf), M_max,
                                       _ptr(y_perm, "y_perm", bf), w, wb, _stream(stream)),
           "moe_expert_ffn_packed")


def moe_expert_ffn_packed_noalloc(x, expert_offset, w1p, w2p, act: int, y_perm, stream=None, row_index=None,
                                  m_max=None):
    """moe_expert_ffn_packed without a workspace argument: the library's
    fixed per-GPU array serves as the workspace (calls overlapping on one GPU
    race on it)."""
    E = expert_offset.numel() - 1
    d = x.shape[1]
    f = w2p.shape[-1]
    M_max = int(m_max if m_max is not None else (y_perm.shape[0] if row_index is not None else x.shape[0]))
    bf = _elem_dtypes(MOE_BF16)
    _check(lib().moe_expert_ffn_packed_noalloc(_ptr(x, "x", bf), int(x.shape[0]),
                                               _ptr(row_index, "row_index", _I32) if row_index is not None else None,
                                               _ptr(expert_offset, "expert_offset", _I32), int(E), int(d), int(f),
                                               int(act), _ptr(w1p, "w1_packed", bf), _ptr(w2p, "w2_packed", bf),
                                               M_max, _ptr(y_perm, "y_perm", bf), _stream(stream)),
           "moe_expert_ffn_packed_noalloc")


def moe_expert_up_packed(x, expert_offset, w1p, act: int, h, ws, stream=None, row_index=None, m_max=None):
    """Up projection + activation on packed weights: h [M_max, f] (bf16).
    row_index / m_max as in moe_expert_ffn_packed; ws: MOE_GEMM_WS_BYTES of
    device memory."""
    E = expert_offset.numel() - 1
    d = x.shape[1]
    f = h.shape[1]
    M_max = int(m_max if m_max is not None else (h.shape[0] if row_index is not None else x.shape[0]))
    bf = _elem_dtypes(MOE_BF16)
    w, wb = _ws(ws)
    _check(lib().moe_expert_up_packed(_ptr(x, "x", bf), int(x.shape[0]),
                                      _ptr(row_index, "row_index", _I32) if row_index is not None else None,
                                      _ptr(expert_offset, "expert_offset", _I32), int(E), int(d), int(f),
                                      int(act), _ptr(w1p, "w1_packed", bf), M_max, _ptr(h, "h", bf), w, wb,
                                      _stream(stream)),
           "moe_expert_up_packed")


def moe_expert_down_packed(h, expert_offset, w2p, y_perm, ws, stream=None, m_max=None):
    """Down projection on packed weights: y_perm = h W2^T per expert."""
    E = expert_offset.numel() - 1
    f = h.shape[1]
    d = y_perm.shape[1]
    M_max = int(m_max if m_max is not None else h.shape[0])
    bf = _elem_dtypes(MOE_BF16)
    w, wb = _ws(ws)
    _check(lib().moe_expert_down_packed(_ptr(h, "h", bf), _ptr(expert_offset, "expert_offset", _I32), int(E),
                                        int(d), int(f), _ptr(w2p, "w2_packed", bf), M_max,
                                        _ptr(y_perm, "y_perm", bf), w, wb, _stream(stream)),
           "moe_expert_down_packed")


def moe_combine(y_perm, rmap: RouteMap, n: int, residual, shared_out, out, stream=None):
    code = dtype_code(y_perm)
    cm = rmap.c()
    _check(lib().moe_combine(_ptr(y_perm, "y_perm", _elem_dtypes(code)), code, ctypes.byref(cm),
                             int(n), int(out.shape[1]), _ptr(residual, "residual", _elem_dtypes(code)),
                             _ptr(shared_out, "shared_out", _elem_dtypes(code)),
                             _ptr(out, "out", _elem_dtypes(code)), _stream(stream)), "moe_combine")


def moe_balance_stats(logits, rmap: RouteMap, cfg: RouteCfg, lb_coef, z_coef, stats, hist=None,
                      ws=None, stream=None):
    w, wb = _ws(ws)
    cm = rmap.c()
    _check(lib().moe_balance_stats(_ptr(logits, "logits", _F32), ctypes.byref(cm), ctypes.byref(cfg),
                                   float(lb_coef), float(z_coef), _ptr(stats, "stats", _F32),
                                   _ptr(hist, "hist", _I32), w, wb, _stream(stream)),
           "moe_balance_stats")


def moe_update_bias(expert_count, cfg: RouteCfg, gamma, bias, stream=None):
    _check(lib().moe_update_bias(_ptr(expert_count, "expert_count", _I32), ctypes.byref(cfg),
                                 float(gamma), _ptr(bias, "bias", _F32), _stream(stream)),
           "moe_update_bias")


# ---------------------------------------------------------------- backward

def moe_combine_backward(dout, y_perm, rmap: RouteMap, dy_perm, d_gate, stream=None):
    code = dtype_code(dout)
    cm = rmap.c()
    el = _elem_dtypes(code)
    _check(lib().moe_combine_backward(_ptr(dout, "dout", el), _ptr(y_perm, "y_perm", el), code,
                                      int(dout.shape[0]), int(dout.shape[1]), ctypes.byref(cm),
                                      int(y_perm.shape[0]), _ptr(dy_perm, "dy_perm", el),
                                      _ptr(d_gate, "d_gate", _F32), _stream(stream)), "moe_combine_backward")


def moe_ffn_backward_workspace_size(M_max: int, E: int, d: int, f: int, act: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_ffn_backward_workspace_size(int(M_max), int(E), int(d), int(f), int(act), int(dtype),
                                                 ctypes.byref(out)), "moe_ffn_backward_workspace_size")
    return out.value


def moe_expert_ffn_backward(x_perm, expert_offset, w1, w2, act: int, dy_perm, dx_perm, dw1, dw2, ws,
                            stream=None):
    """W1 [E, f_rows, d] and W2 [E, d, f] in the natural layout; dW1 and dW2
    fp32 of the same shapes."""
    code = dtype_code(x_perm)
    el = _elem_dtypes(code)
    E = expert_offset.numel() - 1
    d, f = w2.shape[-2], w2.shape[-1]
    w, wb = _ws(ws)
    _check(lib().moe_expert_ffn_backward(_ptr(x_perm, "x_perm", el), code, _ptr(expert_offset, "expert_offset", _I32),
                                         E, d, f, int(act), _ptr(w1, "w1", el), _ptr(w2, "w2", el),
                                         _ptr(dy_perm, "dy_perm", el), int(x_perm.shape[0]),
                                         _ptr(dx_perm, "dx_perm", el), _ptr(dw1, "dw1", _F32),
                                         _ptr(dw2, "dw2", _F32), w, wb, _stream(stream)), "moe_expert_ffn_backward")


def moe_gate_backward(logits, sel_idx, d_gate, cfg: RouteCfg, rmap: RouteMap, lb_coef, z_coef, dz, stream=None):
    cm = rmap.c()
    _check(lib().moe_gate_backward(_ptr(logits, "logits", _F32), _ptr(sel_idx, "sel_idx", _I32),
                                   _ptr(d_gate, "d_gate", _F32), ctypes.byref(cfg), ctypes.byref(cm),
                                   float(lb_coef), float(z_coef), _ptr(dz, "dz", _F32), _stream(stream)),
           "moe_gate_backward")


def moe_router_backward_workspace_size(cfg: RouteCfg, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_router_backward_workspace_size(ctypes.byref(cfg), int(dtype), ctypes.byref(out)),
           "moe_router_backward_workspace_size")
    return out.value


def moe_router_backward(x, wg, dz, cfg: RouteCfg, base, dx, dwg, d_offset, ws, stream=None):
    code = dtype_code(x)
    el = _elem_dtypes(code)
    w, wb = _ws(ws)
    _check(lib().moe_router_backward(_ptr(x, "x", el), _ptr(wg, "wg", el), code, _ptr(dz, "dz", _F32),
                                     ctypes.byref(cfg), _ptr(base, "base", el), _ptr(dx, "dx", el),
                                     _ptr(dwg, "dwg", _F32), _ptr(d_offset, "d_offset", _F32), w, wb,
                                     _stream(stream)), "moe_router_backward")


def moe_dispatch_backward(dx_perm, rmap: RouteMap, n: int, base, base2, dx, stream=None):
    code = dtype_code(dx)
    el = _elem_dtypes(code)
    cm = rmap.c()
    _check(lib().moe_dispatch_backward(_ptr(dx_perm, "dx_perm", el), code, ctypes.byref(cm), int(n),
                                       int(dx.shape[1]), _ptr(base, "base", el), _ptr(base2, "base2", el),
                                       _ptr(dx, "dx", el), _stream(stream)), "moe_dispatch_backward")


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()
