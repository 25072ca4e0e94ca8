// C ABI of the MoE-layer forward: host-side validation, workspace sizing and
// launches.  Every entry point checks its arguments before the first HIP
// call, so argument errors are reported (and testable) without a GPU.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/moe_dispatch.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status_t launched(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(err));
  g_last_error.clear();
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...)                                          \
  do {                                                              \
    if (!(cond)) return fail(MOE_ERR_INVALID_ARG, __VA_ARGS__);     \
  } while (0)
#define SUPPORTED(cond, ...)                                        \
  do {                                                              \
    if (!(cond)) return fail(MOE_ERR_UNSUPPORTED, __VA_ARGS__);     \
  } while (0)

moe_status_t check_cfg(const moe_route_cfg_t* c) {
  REQUIRE(c != nullptr, "cfg is NULL");
  // k = 0 is the degenerate expert choice of a batch too small for any
  // expert to take a token (n c / E rounds to 0)
  REQUIRE(c->n > 0 && c->d > 0 && c->E > 0 && (c->k > 0 || (c->k == 0 && c->dir == MOE_EXPERT_CHOICE)),
          "n, d, E, k must be positive (n=%d d=%d E=%d k=%d; k = 0 only for expert choice)", c->n, c->d,
          c->E, c->k);
  REQUIRE(c->dir == MOE_TOKEN_CHOICE || c->dir == MOE_EXPERT_CHOICE, "dir must be 0 or 1");
  REQUIRE(c->score == MOE_SOFTMAX || c->score == MOE_SIGMOID || c->score == MOE_SQRTSOFTPLUS,
          "score must be MOE_SOFTMAX, MOE_SIGMOID or MOE_SQRTSOFTPLUS");
  REQUIRE(c->capacity_order == MOE_TOKEN_MAJOR || c->capacity_order == MOE_RANK_MAJOR,
          "capacity_order must be MOE_TOKEN_MAJOR or MOE_RANK_MAJOR");
  REQUIRE(c->norm_topk == 0 || c->norm_topk == 1, "norm_topk must be 0 or 1");
  SUPPORTED(c->E <= moe::kMaxExperts, "E=%d exceeds the supported %d experts", c->E, moe::kMaxExperts);
  if (c->dir == MOE_TOKEN_CHOICE) {
    REQUIRE(c->k <= c->E, "token choice needs k <= E (k=%d E=%d)", c->k, c->E);
    SUPPORTED(c->k <= 64, "token choice supports k <= 64 (k=%d)", c->k);
    REQUIRE((int64_t)c->n * c->k <= INT32_MAX, "n*k overflows int32");
    REQUIRE(c->n_group >= 1 && c->E % c->n_group == 0, "E=%d must be a multiple of n_group=%d", c->E,
            c->n_group);
    SUPPORTED(c->n_group <= 64, "n_group <= 64");
    REQUIRE(c->topk_group >= 1 && c->topk_group <= c->n_group, "need 1 <= topk_group <= n_group");
    REQUIRE(c->group_topm >= 1 && c->group_topm <= c->E / c->n_group,
            "need 1 <= group_topm <= experts per group");
    SUPPORTED(c->group_topm <= 4, "group_topm <= 4");
    REQUIRE(c->k <= c->topk_group * (c->E / c->n_group),
            "k=%d exceeds the experts of the %d kept groups", c->k, c->topk_group);
    REQUIRE(c->capacity >= -1, "capacity must be >= -1 (-1 = dropless)");
  } else {
    REQUIRE(c->k <= c->n, "expert choice needs k <= n (k=%d n=%d)", c->k, c->n);
    SUPPORTED(c->score == MOE_SOFTMAX, "expert choice selects on softmax scores");
    REQUIRE(c->capacity_order == MOE_TOKEN_MAJOR, "expert choice has no capacity order");
    SUPPORTED(c->n_group == 1, "expert choice has no group limit");
    SUPPORTED(c->n <= (1 << 24), "expert choice supports n <= 2^24");
    REQUIRE((int64_t)c->E * c->k <= INT32_MAX, "E*k overflows int32");
  }
  return MOE_OK;
}

moe_status_t check_map(const moe_route_map_t* m) {
  REQUIRE(m != nullptr, "map is NULL");
  REQUIRE(m->expert_count && m->expert_offset && m->slot_token && m->slot_gate && m->assign_slot &&
              m->token_offset && m->token_slot && m->n_kept,
          "every routing-map buffer must be non-NULL");
  return MOE_OK;
}

moe::MapPtrs map_ptrs(const moe_route_map_t* m) {
  return moe::MapPtrs{m->expert_count, m->expert_offset, m->slot_token, m->slot_gate,
                      m->assign_slot,  m->token_offset,  m->token_slot, m->n_kept};
}

size_t route_ws(const moe_route_cfg_t* c) {
  size_t b = moe::map_workspace_bytes(c->dir, c->n, c->E, c->k);
  const size_t s = moe::stats_workspace_bytes(c->n, c->E);
  if (s > b) b = s;
  if (c->dir == MOE_EXPERT_CHOICE) {
    const size_t e = moe::select_ec_workspace_bytes(c->n, c->E);
    if (e > b) b = e;
  }
  return b;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int32_t moe_ec_k(int32_t n, double c, int32_t E) {
  if (n <= 0 || E <= 0 || !(c > 0.0)) return -1;
  const double v = std::floor((double)n * c / (double)E + 0.5);
  return v > (double)INT32_MAX ? -1 : (int32_t)v;
}

int32_t moe_tc_capacity(int32_t n, int32_t k, int32_t E, double cf) {
  if (n <= 0 || k <= 0 || E <= 0 || !(cf >= 0.0)) return -1;
  const double v = std::floor(cf * (double)k * (double)n / (double)E + 0.5);
  return v > (double)INT32_MAX ? -1 : (int32_t)v;
}

int64_t moe_max_slots(const moe_route_cfg_t* cfg) {
  if (check_cfg(cfg) != MOE_OK) return -1;
  if (cfg->dir == MOE_EXPERT_CHOICE) return (int64_t)cfg->E * cfg->k;
  const int64_t nk = (int64_t)cfg->n * cfg->k;
  if (cfg->capacity < 0) return nk;
  const int64_t cap = (int64_t)cfg->E * cfg->capacity;
  return cap < nk ? cap : nk;
}

int64_t moe_token_list_len(const moe_route_cfg_t* cfg) {
  if (check_cfg(cfg) != MOE_OK) return -1;
  return cfg->dir == MOE_EXPERT_CHOICE ? (int64_t)cfg->E * cfg->k : (int64_t)cfg->n * cfg->k;
}

moe_status_t moe_router_workspace_size(const moe_route_cfg_t* cfg, int32_t dtype, size_t* bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(bytes != nullptr, "bytes is NULL");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  *bytes = moe::router_workspace_bytes(cfg->n, cfg->d, cfg->E, dtype, cfg->score);
  return MOE_OK;
}

moe_status_t moe_route_workspace_size(const moe_route_cfg_t* cfg, size_t* bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(bytes != nullptr, "bytes is NULL");
  *bytes = route_ws(cfg);
  return MOE_OK;
}

moe_status_t moe_ffn_workspace_size(int64_t M_max, int32_t E, int32_t d, int32_t f, int32_t act,
                                    int32_t dtype, size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is NULL");
  REQUIRE(M_max >= 0 && E > 0 && d > 0 && f > 0, "E, d, f must be positive, M_max non-negative");
  REQUIRE(act == MOE_GELU || act == MOE_SWIGLU, "act must be MOE_GELU or MOE_SWIGLU");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  *bytes = moe::ffn_workspace_bytes(M_max, E, d, f, act, dtype);
  return MOE_OK;
}

moe_status_t moe_router(const void* X, const void* Wg, int32_t dtype, const float* logit_offset,
                        const float* noise, float noise_std, const moe_route_cfg_t* cfg, float* logits,
                        float* scores, float* scores_t, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(X && Wg && logits, "X, Wg and logits must be non-NULL");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  REQUIRE(!noise || std::isfinite(noise_std), "noise_std must be finite");
  if (dtype == MOE_BF16 && cfg->d % 64 == 0 && cfg->E % 16 == 0)   // the matrix-core path
    REQUIRE(aligned16(X) && aligned16(Wg), "X and Wg must be 16-byte aligned");
  const size_t need = moe::router_workspace_bytes(cfg->n, cfg->d, cfg->E, dtype, cfg->score);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "router needs %zu workspace bytes, got %zu", need, ws_bytes);
  return launched(moe::launch_router(X, Wg, dtype, logit_offset, noise, noise ? noise_std : 0.f, cfg->n,
                                     cfg->d, cfg->E, cfg->score, logits, scores, scores_t, ws,
                                     as_stream(stream)),
                  "moe_router");
}

moe_status_t moe_select(const float* logits, const float* scores_t, const float* sel_bias,
                        const moe_route_cfg_t* cfg, int32_t* sel_idx, float* sel_gate, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->k == 0) return MOE_OK;                 // expert choice with nothing to select
  REQUIRE(sel_idx && sel_gate, "sel_idx and sel_gate must be non-NULL");
  if (cfg->dir == MOE_TOKEN_CHOICE) {
    REQUIRE(logits, "logits must be non-NULL");
    moe::SelectArgs a{cfg->n, cfg->E, cfg->k, cfg->score, cfg->n_group, cfg->topk_group,
                      cfg->group_topm, cfg->norm_topk};
    return launched(moe::launch_select_tc(logits, sel_bias, a, sel_idx, sel_gate, as_stream(stream)),
                    "moe_select");
  }
  REQUIRE(logits || scores_t, "expert choice needs logits or scores_t");
  if (!scores_t) {
    const size_t need = moe::select_ec_workspace_bytes(cfg->n, cfg->E);
    if (!ws || ws_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "select needs %zu workspace bytes, got %zu", need, ws_bytes);
  }
  return launched(moe::launch_select_ec(logits, scores_t, cfg->n, cfg->E, cfg->k, sel_idx, sel_gate,
                                        ws, as_stream(stream)),
                  "moe_select");
}

moe_status_t moe_build_map(const int32_t* sel_idx, const float* sel_gate, const moe_route_cfg_t* cfg,
                           const moe_route_map_t* map, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  st = check_map(map);
  if (st != MOE_OK) return st;
  REQUIRE((sel_idx && sel_gate) || cfg->k == 0, "sel_idx and sel_gate must be non-NULL");
  const size_t need = moe::map_workspace_bytes(cfg->dir, cfg->n, cfg->E, cfg->k);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "build_map needs %zu workspace bytes, got %zu", need, ws_bytes);
  const moe::MapPtrs m = map_ptrs(map);
  SUPPORTED((int64_t)cfg->n * cfg->k <= INT32_MAX, "routing maps need n k < 2^31 (n=%d k=%d)", cfg->n, cfg->k);
  if (cfg->dir == MOE_TOKEN_CHOICE)
    return launched(moe::launch_build_map_tc(sel_idx, sel_gate, cfg->n, cfg->E, cfg->k, cfg->capacity,
                                             cfg->capacity_order, m, ws, as_stream(stream)),
                    "moe_build_map");
  return launched(moe::launch_build_map_ec(sel_idx, sel_gate, cfg->n, cfg->E, cfg->k, m, ws,
                                           as_stream(stream)),
                  "moe_build_map");
}

moe_status_t moe_dispatch(const void* X, int32_t dtype, int32_t n, int32_t d, const moe_route_map_t* map,
                          int64_t M_max, void* X_perm, void* stream) {
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  REQUIRE(n > 0 && d > 0 && M_max >= 0, "n, d must be positive, M_max non-negative");
  REQUIRE(M_max <= (int64_t)INT32_MAX * 4, "M_max too large");
  if (M_max == 0) return MOE_OK;                  // no slots: nothing to move
  REQUIRE(X && X_perm, "X and X_perm must be non-NULL");
  REQUIRE(map && map->slot_token && map->n_kept, "map->slot_token and map->n_kept must be non-NULL");
  const int eb = dtype == MOE_BF16 ? 2 : 4;
  if (((int64_t)d * eb) % 16 == 0)
    REQUIRE(aligned16(X) && aligned16(X_perm), "X and X_perm must be 16-byte aligned");
  return launched(moe::launch_dispatch(X, eb, n, d, map->slot_token, map->n_kept, M_max, X_perm,
                                       as_stream(stream)),
                  "moe_dispatch");
}

moe_status_t moe_expert_ffn(const void* X_perm, int32_t dtype, const int32_t* expert_offset, int32_t E,
                            int32_t d, int32_t f, int32_t act, const void* W1, const void* W2,
                            int64_t M_max, void* Y_perm, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(E > 0 && d > 0 && f > 0 && M_max >= 0, "E, d, f must be positive, M_max non-negative");
  if (M_max == 0) return MOE_OK;                  // no rows: nothing to compute
  REQUIRE(X_perm && expert_offset && W1 && W2 && Y_perm, "tensor arguments must be non-NULL");
  REQUIRE(act == MOE_GELU || act == MOE_SWIGLU, "act must be MOE_GELU or MOE_SWIGLU");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  REQUIRE(M_max <= INT32_MAX, "M_max must fit in int32");
  if (dtype == MOE_BF16) {
    SUPPORTED(E <= moe::kMaxExperts, "bf16 expert FFN supports E <= %d (E=%d)", moe::kMaxExperts, E);
    SUPPORTED(d % 64 == 0 && f % 64 == 0, "bf16 expert FFN needs d %% 64 == 0 and f %% 64 == 0 (d=%d f=%d)",
              d, f);
    REQUIRE(aligned16(X_perm) && aligned16(W1) && aligned16(W2) && aligned16(Y_perm),
            "bf16 tensors must be 16-byte aligned");
  }
  const size_t need = moe::ffn_workspace_bytes(M_max, E, d, f, act, dtype);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "expert_ffn needs %zu workspace bytes, got %zu", need, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  return launched(moe::launch_expert_ffn(X_perm, nullptr, 0, dtype, expert_offset, E, d, f, act, W1, W2,
                                         M_max, Y_perm, ws, false, as_stream(stream)),
                  "moe_expert_ffn");
}

moe_status_t moe_pack_expert_weights(const void* W, int32_t E, int32_t rows, int32_t K, int32_t gate_up,
                                     void* W_packed, void* stream) {
  REQUIRE(W && W_packed, "W and W_packed must be non-NULL");
  REQUIRE(W != W_packed, "W_packed must not alias W");
  REQUIRE(E > 0 && rows > 0 && K > 0, "E, rows, K must be positive");
  REQUIRE(gate_up == 0 || gate_up == 1, "gate_up must be 0 or 1");
  SUPPORTED(rows % (gate_up ? 64 : 32) == 0 && K % 64 == 0,
            "packing needs rows %% 32 == 0 (gate_up: rows %% 64 == 0) and K %% 64 == 0 (rows=%d K=%d)", rows, K);
  REQUIRE(aligned16(W) && aligned16(W_packed), "W and W_packed must be 16-byte aligned");
  return launched(moe::launch_pack_weights(W, E, rows, K, gate_up, W_packed, as_stream(stream)),
                  "moe_pack_expert_weights");
}

// Arguments of the packed FFN other than its workspace (M_max > 0).
static moe_status_t check_ffn_packed(const void* X, int32_t n_x, const int32_t* row_index,
                                     const int32_t* expert_offset, int32_t E, int32_t d, int32_t f, int32_t act,
                                     const void* W1_packed, const void* W2_packed, int64_t M_max,
                                     void* Y_perm) {
  REQUIRE(X && expert_offset && W1_packed && W2_packed && Y_perm, "tensor arguments must be non-NULL");
  REQUIRE(!row_index || n_x > 0, "n_x must be positive when row_index is given");
  REQUIRE(act == MOE_GELU || act == MOE_SWIGLU, "act must be MOE_GELU or MOE_SWIGLU");
  REQUIRE(M_max <= INT32_MAX, "M_max must fit in int32");
  SUPPORTED(E <= moe::kMaxExperts, "bf16 expert FFN supports E <= %d (E=%d)", moe::kMaxExperts, E);
  SUPPORTED(d % 64 == 0 && f % 64 == 0, "bf16 expert FFN needs d %% 64 == 0 and f %% 64 == 0 (d=%d f=%d)",
            d, f);
  REQUIRE(aligned16(X) && aligned16(W1_packed) && aligned16(W2_packed) && aligned16(Y_perm),
          "bf16 tensors must be 16-byte aligned");
  return MOE_OK;
}

moe_status_t moe_expert_ffn_packed_noalloc(const void* X, int32_t n_x, const int32_t* row_index,
                                           const int32_t* expert_offset, int32_t E, int32_t d, int32_t f,
                                           int32_t act, const void* W1_packed, const void* W2_packed,
                                           int64_t M_max, void* Y_perm, void* stream) {
  REQUIRE(E > 0 && d > 0 && f > 0 && M_max >= 0, "E, d, f must be positive, M_max non-negative");
  if (M_max == 0) return MOE_OK;                  // no rows: nothing to compute
  moe_status_t st = check_ffn_packed(X, n_x, row_index, expert_offset, E, d, f, act, W1_packed, W2_packed,
                                     M_max, Y_perm);
  if (st != MOE_OK) return st;
  const size_t need = moe::ffn_workspace_bytes(M_max, E, d, f, act, MOE_BF16);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_expert_ffn_packed_noalloc: M_max x f = %lld x %d needs %zu bytes of workspace, more than "
                "its fixed %d-byte array; use moe_expert_ffn_packed with a caller workspace",
                (long long)M_max, f, need, (int)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t err = moe::noalloc_scratch(&ws);
  if (err != hipSuccess)
    return fail(MOE_ERR_LAUNCH, "moe_expert_ffn_packed_noalloc: the library's workspace array: %s",
                hipGetErrorString(err));
  return launched(moe::launch_expert_ffn(X, row_index, n_x, MOE_BF16, expert_offset, E, d, f, act, W1_packed,
                                         W2_packed, M_max, Y_perm, ws, true, as_stream(stream)),
                  "moe_expert_ffn_packed_noalloc");
}

moe_status_t moe_expert_ffn_packed(const void* X, int32_t n_x, const int32_t* row_index,
                                   const int32_t* expert_offset, int32_t E, int32_t d, int32_t f, int32_t act,
                                   const void* W1_packed, const void* W2_packed, int64_t M_max, void* Y_perm,
                                   void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(E > 0 && d > 0 && f > 0 && M_max >= 0, "E, d, f must be positive, M_max non-negative");
  if (M_max == 0) return MOE_OK;                  // no rows: nothing to compute
  moe_status_t st = check_ffn_packed(X, n_x, row_index, expert_offset, E, d, f, act, W1_packed, W2_packed,
                                     M_max, Y_perm);
  if (st != MOE_OK) return st;
  const size_t need = moe::ffn_workspace_bytes(M_max, E, d, f, act, MOE_BF16);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "expert_ffn needs %zu workspace bytes, got %zu", need, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  return launched(moe::launch_expert_ffn(X, row_index, n_x, MOE_BF16, expert_offset, E, d, f, act, W1_packed,
                                         W2_packed, M_max, Y_perm, ws, true, as_stream(stream)),
                  "moe_expert_ffn_packed");
}

// Shape rules shared by the packed FFN calls.
static moe_status_t check_packed_ffn(int32_t E, int32_t d, int32_t f, int64_t M_max) {
  REQUIRE(E > 0 && d > 0 && f > 0 && M_max >= 0, "E, d, f must be positive, M_max non-negative");
  REQUIRE(M_max <= INT32_MAX, "M_max must fit in int32");
  SUPPORTED(E <= moe::kMaxExperts, "bf16 expert FFN supports E <= %d (E=%d)", moe::kMaxExperts, E);
  SUPPORTED(d % 64 == 0 && f % 64 == 0, "bf16 expert FFN needs d %% 64 == 0 and f %% 64 == 0 (d=%d f=%d)",
            d, f);
  return MOE_OK;
}

static_assert(MOE_GEMM_WS_BYTES == moe::kGemmWsBytes, "header and kernels agree on the GEMM workspace");

static moe_status_t check_gemm_ws(void* ws, size_t ws_bytes, const char* who) {
  if (!ws || ws_bytes < MOE_GEMM_WS_BYTES)
    return fail(MOE_ERR_WORKSPACE, "%s needs %d workspace bytes, got %zu", who, (int)MOE_GEMM_WS_BYTES, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  return MOE_OK;
}

moe_status_t moe_expert_up_packed(const void* X, int32_t n_x, const int32_t* row_index,
                                  const int32_t* expert_offset, int32_t E, int32_t d, int32_t f, int32_t act,
                                  const void* W1_packed, int64_t M_max, void* H, void* ws, size_t ws_bytes,
                                  void* stream) {
  moe_status_t st = check_packed_ffn(E, d, f, M_max);
  if (st != MOE_OK) return st;
  if (M_max == 0) return MOE_OK;
  REQUIRE(X && expert_offset && W1_packed && H, "tensor arguments must be non-NULL");
  REQUIRE(!row_index || n_x > 0, "n_x must be positive when row_index is given");
  REQUIRE(act == MOE_GELU || act == MOE_SWIGLU, "act must be MOE_GELU or MOE_SWIGLU");
  REQUIRE(aligned16(X) && aligned16(W1_packed) && aligned16(H), "bf16 tensors must be 16-byte aligned");
  REQUIRE(H != X, "H must not alias X");
  if ((st = check_gemm_ws(ws, ws_bytes, "moe_expert_up_packed")) != MOE_OK) return st;
  return launched(moe::launch_expert_gemm(1, X, row_index, n_x, expert_offset, E, d, f, act, W1_packed, M_max, H,
                                          true, ws, as_stream(stream)),
                  "moe_expert_up_packed");
}

moe_status_t moe_expert_down_packed(const void* H, const int32_t* expert_offset, int32_t E, int32_t d, int32_t f,
                                    const void* W2_packed, int64_t M_max, void* Y_perm, void* ws, size_t ws_bytes,
                                    void* stream) {
  moe_status_t st = check_packed_ffn(E, d, f, M_max);
  if (st != MOE_OK) return st;
  if (M_max == 0) return MOE_OK;
  REQUIRE(H && expert_offset && W2_packed && Y_perm, "tensor arguments must be non-NULL");
  REQUIRE(aligned16(H) && aligned16(W2_packed) && aligned16(Y_perm), "bf16 tensors must be 16-byte aligned");
  REQUIRE(H != Y_perm, "Y_perm must not alias H");
  if ((st = check_gemm_ws(ws, ws_bytes, "moe_expert_down_packed")) != MOE_OK) return st;
  return launched(moe::launch_expert_gemm(2, H, nullptr, (int)M_max, expert_offset, E, d, f, MOE_GELU, W2_packed,
                                          M_max, Y_perm, true, ws, as_stream(stream)),
                  "moe_expert_down_packed");
}

moe_status_t moe_combine(const void* Y_perm, int32_t dtype, const moe_route_map_t* map, int32_t n,
                         int32_t d, const void* residual, const void* shared_out, void* out,
                         void* stream) {
  REQUIRE(Y_perm && out, "Y_perm and out must be non-NULL");
  REQUIRE(map && map->token_offset && map->token_slot && map->slot_gate,
          "map->token_offset, token_slot and slot_gate must be non-NULL");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  REQUIRE(n > 0 && d > 0, "n, d must be positive");
  REQUIRE(out != Y_perm && out != residual && out != shared_out, "out must not alias an input");
  const int vec = dtype == MOE_BF16 ? 8 : 4;
  if (d % vec == 0)
    REQUIRE(aligned16(Y_perm) && aligned16(out) && (!residual || aligned16(residual)) &&
                (!shared_out || aligned16(shared_out)),
            "tensors must be 16-byte aligned");
  return launched(moe::launch_combine(Y_perm, dtype, map->token_offset, map->token_slot, map->slot_gate, n,
                                      d, residual, shared_out, out, as_stream(stream)),
                  "moe_combine");
}

moe_status_t moe_balance_stats(const float* logits, const moe_route_map_t* map,
                               const moe_route_cfg_t* cfg, float lb_coef, float z_coef, float* stats,
                               int32_t* hist, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(logits && stats, "logits and stats must be non-NULL");
  REQUIRE(map && map->expert_count && map->expert_offset && map->token_offset && map->token_slot,
          "map->expert_count, expert_offset and token_offset must be non-NULL");
  const size_t need = moe::stats_workspace_bytes(cfg->n, cfg->E);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "balance_stats needs %zu workspace bytes, got %zu", need, ws_bytes);
  return launched(moe::launch_balance_stats(logits, map_ptrs(map), cfg->n, cfg->E, cfg->k, cfg->dir,
                                            cfg->score, lb_coef, z_coef, stats, hist, ws,
                                            as_stream(stream)),
                  "moe_balance_stats");
}

moe_status_t moe_update_bias(const int32_t* expert_count, const moe_route_cfg_t* cfg, float gamma,
                             float* bias, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(cfg->dir == MOE_TOKEN_CHOICE, "the bias update balances token choice (expert choice loads are fixed)");
  REQUIRE(expert_count && bias, "expert_count and bias must be non-NULL");
  REQUIRE(std::isfinite(gamma), "gamma must be finite");
  return launched(moe::launch_update_bias(expert_count, cfg->n, cfg->E, cfg->k, gamma, bias,
                                          as_stream(stream)),
                  "moe_update_bias");
}

// ---- backward -----------------------------------------------------------

moe_status_t moe_combine_backward(const void* dOut, const void* Y_perm, int32_t dtype, int32_t n, int32_t d,
                                  const moe_route_map_t* map, int64_t M_max, void* dY_perm, float* d_gate,
                                  void* stream) {
  REQUIRE(n > 0 && d > 0 && M_max >= 0, "n, d must be positive, M_max non-negative");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  if (M_max == 0) return MOE_OK;
  REQUIRE(M_max <= INT32_MAX, "M_max must fit in int32");
  REQUIRE(dOut && Y_perm && dY_perm && d_gate, "tensor arguments must be non-NULL");
  REQUIRE(map && map->slot_token && map->slot_gate && map->n_kept,
          "map->slot_token, slot_gate and n_kept must be non-NULL");
  REQUIRE(dY_perm != Y_perm && dY_perm != dOut, "dY_perm must not alias an input");
  if (dtype == MOE_BF16 && d % 8 == 0)
    REQUIRE(aligned16(dOut) && aligned16(Y_perm) && aligned16(dY_perm), "tensors must be 16-byte aligned");
  return launched(moe::launch_combine_backward(dOut, Y_perm, dtype, d, map->slot_token, map->slot_gate,
                                               map->n_kept, M_max, dY_perm, d_gate, as_stream(stream)),
                  "moe_combine_backward");
}

moe_status_t moe_ffn_backward_workspace_size(int64_t M_max, int32_t E, int32_t d, int32_t f, int32_t act,
                                             int32_t dtype, size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is NULL");
  REQUIRE(M_max >= 0 && E > 0 && d > 0 && f > 0, "E, d, f must be positive, M_max non-negative");
  REQUIRE(act == MOE_GELU || act == MOE_SWIGLU, "act must be MOE_GELU or MOE_SWIGLU");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  *bytes = moe::ffn_backward_workspace_bytes(M_max, E, d, f, act, dtype);
  return MOE_OK;
}

moe_status_t moe_expert_ffn_backward(const void* X_perm, int32_t dtype, const int32_t* expert_offset, int32_t E,
                                     int32_t d, int32_t f, int32_t act, const void* W1, const void* W2,
                                     const void* dY_perm, int64_t M_max, void* dX_perm, float* dW1, float* dW2,
                                     void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(E > 0 && d > 0 && f > 0 && M_max >= 0, "E, d, f must be positive, M_max non-negative");
  REQUIRE(act == MOE_GELU || act == MOE_SWIGLU, "act must be MOE_GELU or MOE_SWIGLU");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  REQUIRE(expert_offset && W1 && W2 && dW1 && dW2, "expert_offset, W1, W2, dW1 and dW2 must be non-NULL");
  REQUIRE(M_max == 0 || (X_perm && dY_perm && dX_perm), "X_perm, dY_perm and dX_perm must be non-NULL");
  REQUIRE(M_max <= INT32_MAX, "M_max must fit in int32");
  SUPPORTED(E <= moe::kMaxExperts, "expert FFN backward supports E <= %d (E=%d)", moe::kMaxExperts, E);
  const int64_t fr = act == MOE_SWIGLU ? 2 * (int64_t)f : f;
  // the bf16 kernels address every operand and the fp32 weight gradients
  // through 32-bit byte offsets
  REQUIRE(M_max * fr <= INT32_MAX / 4 && M_max * (int64_t)d <= INT32_MAX / 4 && fr * d <= INT32_MAX / 4,
          "M_max x width and the weight matrices must have fewer than 2^29 elements");
  REQUIRE(aligned16(dW1) && aligned16(dW2), "dW1 and dW2 must be 16-byte aligned");
  if (dtype == MOE_BF16)
    REQUIRE(aligned16(W1) && aligned16(W2) && (M_max == 0 || (aligned16(X_perm) && aligned16(dY_perm) &&
                                                              aligned16(dX_perm))),
            "bf16 tensors must be 16-byte aligned");
  const size_t need = moe::ffn_backward_workspace_bytes(M_max, E, d, f, act, dtype);
  if (need && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "expert_ffn_backward needs %zu workspace bytes, got %zu", need, ws_bytes);
  REQUIRE(!need || aligned16(ws), "workspace must be 16-byte aligned");
  return launched(moe::launch_expert_ffn_backward(X_perm, dtype, expert_offset, E, d, f, act, W1, W2, dY_perm,
                                                  M_max, dX_perm, dW1, dW2, ws, as_stream(stream)),
                  "moe_expert_ffn_backward");
}

moe_status_t moe_gate_backward(const float* logits, const int32_t* sel_idx, const float* d_gate,
                               const moe_route_cfg_t* cfg, const moe_route_map_t* map, float lb_coef,
                               float z_coef, float* dZ, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  st = check_map(map);
  if (st != MOE_OK) return st;
  REQUIRE(logits && dZ, "logits and dZ must be non-NULL");
  REQUIRE(cfg->k == 0 || d_gate, "d_gate must be non-NULL");
  REQUIRE(cfg->dir == MOE_EXPERT_CHOICE || sel_idx, "token choice needs sel_idx");
  REQUIRE(std::isfinite(lb_coef) && std::isfinite(z_coef), "coefficients must be finite");
  return launched(moe::launch_gate_backward(logits, sel_idx, d_gate, map_ptrs(map), cfg->n, cfg->E, cfg->k,
                                            cfg->dir, cfg->score, cfg->norm_topk, lb_coef, z_coef, dZ,
                                            as_stream(stream)),
                  "moe_gate_backward");
}

moe_status_t moe_router_backward_workspace_size(const moe_route_cfg_t* cfg, int32_t dtype, size_t* bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(bytes != nullptr, "bytes is NULL");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  *bytes = moe::router_backward_workspace_bytes(cfg->n, cfg->d, cfg->E, dtype);
  return MOE_OK;
}

moe_status_t moe_router_backward(const void* X, const void* Wg, int32_t dtype, const float* dZ,
                                 const moe_route_cfg_t* cfg, const void* base, void* dX, float* dWg,
                                 float* d_offset, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  REQUIRE(X && Wg && dZ, "X, Wg and dZ must be non-NULL");
  REQUIRE(!dX || (dX != X && dX != base), "dX must not alias X or base");
  REQUIRE((int64_t)cfg->n * cfg->d <= INT32_MAX && (int64_t)cfg->d * cfg->E <= INT32_MAX,
          "n x d and d x E must have fewer than 2^31 elements");
  if (dtype == MOE_BF16)
    REQUIRE(aligned16(X) && aligned16(Wg) && (!dX || aligned16(dX)) && (!base || aligned16(base)),
            "bf16 tensors must be 16-byte aligned");
  const size_t need = moe::router_backward_workspace_bytes(cfg->n, cfg->d, cfg->E, dtype);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "router_backward needs %zu workspace bytes, got %zu", need, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  return launched(moe::launch_router_backward(X, Wg, dtype, dZ, cfg->n, cfg->d, cfg->E, base, dX, dWg,
                                              d_offset, ws, as_stream(stream)),
                  "moe_router_backward");
}

moe_status_t moe_dispatch_backward(const void* dX_perm, int32_t dtype, const moe_route_map_t* map, int32_t n,
                                   int32_t d, const void* base, const void* base2, void* dX, void* stream) {
  REQUIRE(dX_perm && dX, "dX_perm and dX must be non-NULL");
  REQUIRE(map && map->token_offset && map->token_slot, "map->token_offset and token_slot must be non-NULL");
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, "dtype must be MOE_F32 or MOE_BF16");
  REQUIRE(n > 0 && d > 0, "n, d must be positive");
  REQUIRE(dX != dX_perm && dX != base && dX != base2, "dX must not alias an input");
  const int vec = dtype == MOE_BF16 ? 8 : 4;
  if (d % vec == 0)
    REQUIRE(aligned16(dX_perm) && aligned16(dX) && (!base || aligned16(base)) && (!base2 || aligned16(base2)),
            "tensors must be 16-byte aligned");
  return launched(moe::launch_combine(dX_perm, dtype, map->token_offset, map->token_slot, nullptr, n, d, base,
                                      base2, dX, as_stream(stream)),
                  "moe_dispatch_backward");
}

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
