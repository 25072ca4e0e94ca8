/*
 * moe_dispatch.h -- C ABI of a Mixture-of-Experts layer forward, and its
 * backward, on one AMD Instinct MI355X (gfx950).
 *
 * The layer (MoE-routing pages: page 2 "Expert choice routing", section "The
 * math"; page 5 "MoE routing strategies explained", strategies 1-6):
 *
 *   S = softmax(X W_g), sigmoid or sqrtsoftplus         moe_router
 *   token choice: each token keeps its top-k experts;   moe_select
 *   expert choice: each expert keeps its top-k tokens
 *   capacity / routing map (P = onehot(I))              moe_build_map
 *   X_in[e] = P[e] X                                    moe_dispatch
 *   Y[e] = Expert_e(X_in[e])                            moe_expert_ffn
 *     (bf16, packed weights, dispatch fused in)         moe_pack_expert_weights,
 *                                                       moe_expert_ffn_packed
 *     (its up and down projections one by one)          moe_expert_up_packed,
 *                                                       moe_expert_down_packed
 *   out = residual + shared + scatter_add(G * Y, I)     moe_combine
 *   load-balance loss, z-loss, MaxVio                   moe_balance_stats
 *   loss-free balancing: bias step from the loads       moe_update_bias
 *
 * The backward (gradients of <dOut, out> + the auxiliary losses, routing
 * fixed), each step reversed:
 *   dY = G * dOut[I], dG = <dOut[I], Y>                 moe_combine_backward
 *   dX_in, dW1, dW2 of the expert FFNs                  moe_expert_ffn_backward
 *   dZ from dG and the auxiliary losses                 moe_gate_backward
 *   dX += dZ W_g^T, dW_g = X^T dZ                       moe_router_backward
 *   dX += P^T dX_in                                     moe_dispatch_backward
 *
 * Conventions common to every call:
 *  - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *    allocates no device memory; calls that need scratch space take a
 *    caller-owned workspace (`ws`, `ws_bytes`) whose size the *_workspace_size
 *    queries give.  Configuration structs are HOST pointers, read during the
 *    call only.
 *  - Every call validates its arguments on the host before touching the GPU
 *    and returns MOE_ERR_INVALID_ARG (bad shape, null pointer, k > E, ...),
 *    MOE_ERR_UNSUPPORTED (a valid request the library does not implement) or
 *    MOE_ERR_WORKSPACE (workspace too small) without any device work.  A HIP
 *    launch failure returns MOE_ERR_LAUNCH.  moe_last_error() returns a
 *    thread-local message for the last non-OK status.  No exception or abort
 *    crosses the ABI.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream).  Results are valid once the stream
 *    has synchronised.  No call synchronises the host with the device: sizes
 *    that depend on routing (per-expert counts, kept assignments) stay on the
 *    device, and host-side buffer sizes use the bounds below.
 *  - Layouts are row-major.  bf16 tensors are raw bfloat16 bit patterns
 *    (uint16) rounded to nearest-even; fp32 tensors are IEEE float.  Expert
 *    weights are K-contiguous: W1 [E, f, d] (SwiGLU: [E, 2f, d], gate rows
 *    first, then up rows), W2 [E, d, f].  The router weight keeps the pages'
 *    [d, E] layout.
 *  - Inputs must be finite.  Results are deterministic: the same inputs give
 *    the same bits on every run (no floating-point atomics).
 *  - A tensor argument of zero elements may be any non-NULL address (it is
 *    never dereferenced); moe_dispatch and moe_expert_ffn with M_max = 0
 *    return MOE_OK at once and ignore their tensor arguments.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_LAUNCH = 4
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };               /* element type           */
enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1, MOE_SQRTSOFTPLUS = 2 };   /* router score function */
enum { MOE_TOKEN_MAJOR = 0, MOE_RANK_MAJOR = 1 }; /* capacity arrival order */
enum { MOE_TOKEN_CHOICE = 0, MOE_EXPERT_CHOICE = 1 };
enum { MOE_GELU = 0, MOE_SWIGLU = 1 };            /* expert activation      */

#define MOE_NSTATS 8
/* moe_balance_stats output, in this order:
 *  0 lb_loss   = lb_coef * E * sum_e f_e * P_e  (f_e: share of chosen
 *                assignments before drops; P_e: mean normalised score)
 *  1 z_loss    = z_coef * mean_t logsumexp(z_t)^2
 *  2 max_vio   = (max_e load_e - mean load) / mean load, load = kept rows
 *  3 max_load_share = max_e load_e / total kept (router-collapse flag)
 *  4 kept assignments         5 dropped assignments
 *  6 tokens with no kept expert (dropped entirely / selected by no expert)
 *  7 largest number of experts any token kept                            */

/* Routing configuration (host struct). */
typedef struct {
  int32_t n;          /* tokens                                            */
  int32_t d;          /* model dimension                                   */
  int32_t E;          /* experts                                           */
  int32_t k;          /* token choice: experts per token; expert choice:
                         tokens per expert (see moe_ec_k)                  */
  int32_t dir;        /* MOE_TOKEN_CHOICE | MOE_EXPERT_CHOICE              */
  int32_t score;      /* MOE_SOFTMAX | MOE_SIGMOID (token choice only)     */
  int32_t n_group;    /* group-limited routing: contiguous expert groups;
                         1 = no group limit                                */
  int32_t topk_group; /* groups kept per token (1 <= topk_group <= n_group) */
  int32_t group_topm; /* group score = sum of the group's top-m keys, 1..4  */
  int32_t norm_topk;  /* 1: renormalise gates over the k selected experts  */
  int32_t capacity;   /* token choice: slots per expert; -1 = dropless     */
  int32_t capacity_order; /* token choice: MOE_TOKEN_MAJOR (assignments arrive
                         token by token, each token's in rank order) or
                         MOE_RANK_MAJOR (every token's first choice arrives
                         before any second choice); expert choice: 0       */
} moe_route_cfg_t;

/* Routing map (host struct of caller-owned device buffers; M_max =
 * moe_max_slots(cfg)).  Slots are expert-major: expert e owns slots
 * expert_offset[e] .. expert_offset[e+1]-1, filled in arrival order. */
typedef struct {
  int32_t *expert_count;  /* [E]   assignments chosen per expert (pre-drop) */
  int32_t *expert_offset; /* [E+1] exclusive prefix of kept rows per expert */
  int32_t *slot_token;    /* [M_max] token of each slot                      */
  float   *slot_gate;     /* [M_max] gate of each slot                       */
  int32_t *assign_slot;   /* token choice [n,k]: slot of (token, rank), -1 =
                             dropped; expert choice [E,k]: slot of I[e,j]   */
  int32_t *token_offset;  /* [n+1] token t's list is token_slot[token_offset[t]
                             .. token_offset[t+1]-1]                        */
  int32_t *token_slot;    /* [moe_token_list_len] token choice: the token's k
                             slots in rank order, -1 where dropped
                             (token_offset[t] = t*k); expert choice: the
                             slots of the experts that picked the token, in
                             ascending expert order                         */
  int32_t *n_kept;        /* [1]   kept assignments = expert_offset[E]       */
} moe_route_map_t;

/* ---- sizes (pure host functions, no GPU needed) ---------------------- */

/* Tokens per expert under expert choice, k = n c / E (page 1 "Who picks
 * whom"; page 2 "A worked example"), rounded half up.  Returns -1 on
 * invalid input (n, E <= 0, c <= 0).  A batch with n c / E < 1/2 gets
 * k = 0, which every call accepts for expert choice: no expert takes a
 * token, the map has no slots (M_max = 0; moe_dispatch and moe_expert_ffn
 * do nothing), and the combine returns the residual plus the shared expert. */
int32_t moe_ec_k(int32_t n, double c, int32_t E);

/* Per-expert capacity under token choice: cf * k * n / E (the balanced load
 * times the capacity factor; page 5 strategy 2 states it for k = 1), rounded
 * half up, computed in double as ((cf * k) * n) / E.  -1 on invalid input. */
int32_t moe_tc_capacity(int32_t n, int32_t k, int32_t E, double cf);

/* Upper bound on kept assignments: token choice n*k (capacity-limited:
 * min(n*k, E*capacity)); expert choice E*k.  -1 on invalid cfg. */
int64_t moe_max_slots(const moe_route_cfg_t *cfg);

/* Length of the token-side list (map->token_slot): n*k under token choice
 * (dropped assignments keep a -1 entry), E*k under expert choice.  -1 on
 * invalid cfg. */
int64_t moe_token_list_len(const moe_route_cfg_t *cfg);

/* Workspace for moe_router (`dtype` of X and W_g). */
moe_status_t moe_router_workspace_size(const moe_route_cfg_t *cfg, int32_t dtype, size_t *bytes);
/* Workspace shared by moe_select, moe_build_map and moe_balance_stats. */
moe_status_t moe_route_workspace_size(const moe_route_cfg_t *cfg, size_t *bytes);
/* Workspace for moe_expert_ffn with M_max rows and hidden size f. */
moe_status_t moe_ffn_workspace_size(int64_t M_max, int32_t E, int32_t d, int32_t f, int32_t act,
                                    int32_t dtype, size_t *bytes);

/* ---- the layer --------------------------------------------------------- */

/* Router (page 2 "The math": S = softmax(X W_g), W_g: [d, E]; page 5
 * strategy 4: a sigmoid per expert instead, or sqrtsoftplus(z) =
 * sqrt(log(1 + e^z)) for DeepSeek-V4).  Logits Z = X W_g accumulated in fp32
 * (bf16 inputs on the matrix cores), plus logit_offset[e] when given, plus
 * noise_std * noise[t,e] when `noise` is given (noisy top-k, page 4 "How MoE
 * routing strategies make LLMs efficient", section "Pitfalls": Gaussian
 * noise on the gating logits; `noise` [n,E] fp32 holds the caller's
 * standard normals, one fp32 multiply and one add), written to logits [n,E]
 * fp32; everything downstream sees these logits.  Optional outputs: scores
 * [n,E] and
 * scores_t [E,n] (the transpose, the column-contiguous layout expert choice
 * selects from), both fp32, computed with the library's specified exp
 * (Cody-Waite reduction, degree-7 Taylor polynomial, single fp32 operations,
 * no fused multiply-add), a halving-stride tree sum over experts and IEEE
 * division, so equal logits give equal score bits on any conforming device
 * (sqrtsoftplus: max(z,0) + log1p(spec_exp(-|z|)), log1p as a specified
 * degree-15 odd series in u/(2+u), then the correctly rounded square root).
 * X [n,d] and W_g [d,E] in `dtype`; logit_offset [E] fp32 or NULL.
 * Any shape; bf16 with d % 64 == 0 and E % 16 == 0 runs on the matrix cores
 * (X and W_g 16-byte aligned), other shapes on a scalar fp32 kernel. */
moe_status_t moe_router(const void *X, const void *Wg, int32_t dtype, const float *logit_offset,
                        const float *noise, float noise_std, const moe_route_cfg_t *cfg,
                        float *logits, float *scores, float *scores_t, void *ws, size_t ws_bytes,
                        void *stream);

/* Selection.
 * Token choice (page 2 "Token-choice and its load-balance headache"; page 5
 * strategies 1, 2, 4, 5): every token keeps its k best experts, in rank
 * order, lower expert index first on equal keys.  Key = the logit (softmax
 * is monotone within a row) or score(z) + sel_bias[e] for the sigmoid and
 * sqrtsoftplus scores (sel_bias [E] fp32 or NULL; the bias enters the
 * choice only).  With n_group > 1 the experts
 * form n_group contiguous groups, each scored by the sum of its top
 * group_topm keys, and only the topk_group best groups (lower index on ties)
 * stay eligible.  Gates: softmax over the k selected logits when norm_topk,
 * else the full-row softmax probability; sigmoid / sqrtsoftplus: the raw
 * scores, renormalised over the k when norm_topk.  Output sel_idx [n,k] int32,
 * sel_gate [n,k] fp32.
 * Expert choice (page 2 "The transposed selection"): every expert keeps the
 * k tokens with the highest softmax score in its column, lower token index
 * first on equal scores; I [E,k] int32 in ascending token order, G [E,k] =
 * S[I, e].  scores_t [E,n] from moe_router is used when given, else it is
 * recomputed from `logits` into the workspace.  n <= 2^24. */
moe_status_t moe_select(const float *logits, const float *scores_t, const float *sel_bias,
                        const moe_route_cfg_t *cfg, int32_t *sel_idx, float *sel_gate, void *ws,
                        size_t ws_bytes, void *stream);

/* Routing map.  Token choice: assignments arrive in token order and, within
 * a token, in rank order (cfg->capacity_order MOE_TOKEN_MAJOR), or rank by
 * rank, tokens in order within a rank (MOE_RANK_MAJOR: first choices have
 * priority); an assignment is kept iff fewer than `capacity` earlier
 * arrivals went to its expert (page 1 "Dropped tokens flow in opposite
 * directions": an assignment that reaches a full buffer is not computed,
 * its token keeps the residual); capacity -1 keeps all (dropless).
 * Expert choice: slot e*k + j holds I[e,j].  Fills every field of `map`;
 * kept slots are expert-major and in arrival order within an expert. */
moe_status_t moe_build_map(const int32_t *sel_idx, const float *sel_gate, const moe_route_cfg_t *cfg,
                           const moe_route_map_t *map, void *ws, size_t ws_bytes, void *stream);

/* Dispatch X_in = P X (page 2 "The math"): X_perm[s] = X[slot_token[s]]
 * for s < n_kept (read on the device); rows n_kept..M_max-1 are left
 * untouched.  X [n,d], X_perm [M_max,d] in `dtype`. */
moe_status_t moe_dispatch(const void *X, int32_t dtype, int32_t n, int32_t d,
                          const moe_route_map_t *map, int64_t M_max, void *X_perm, void *stream);

/* Expert FFNs as one grouped GEMM (page 2 "The math": Y[e] =
 * Expert_e(X_in[e]) on dense per-expert batches).  Rows
 * expert_offset[e] .. expert_offset[e+1]-1 (device array [E+1]) of X_perm
 * go through expert e: GELU: Y = gelu(X W1_e^T) W2_e^T; SwiGLU:
 * Y = (silu(X Wg_e^T) * (X Wu_e^T)) W2_e^T.  bf16: fp32 accumulation on the
 * matrix cores, the hidden activation rounded to bf16, d % 64 == 0 and
 * f % 64 == 0.  fp32: fp32 throughout, any shape.  The always-on shared
 * expert of page 5 strategy 3 is the same call with E = 1 and offsets
 * {0, n}.  Rows >= expert_offset[E] of Y_perm are left untouched. */
moe_status_t moe_expert_ffn(const void *X_perm, int32_t dtype, const int32_t *expert_offset,
                            int32_t E, int32_t d, int32_t f, int32_t act, const void *W1,
                            const void *W2, int64_t M_max, void *Y_perm, void *ws, size_t ws_bytes,
                            void *stream);

/* Packed expert weights: the same bf16 values in the order the matrix cores
 * consume them, so that the expert FFN reads every weight tile as whole
 * contiguous blocks (the FFN of page 2 "The math" streams every expert's
 * weights from memory once per call; this is a one-time layout change of
 * the stored weights, done when they are loaded).  W [E, rows, K] (bf16,
 * K-contiguous) -> W_packed, same size:
 *   row block p of expert e = 32 rows: rows 32p .. 32p+31; with gate_up = 1
 *   (a SwiGLU W1, rows = 2f, gate rows first) block 2q holds the gate rows
 *   32q .. 32q+31 and block 2q+1 the up rows f+32q .. f+32q+31;
 *   a 1 KB chunk holds, at 16-byte slot l (l = 0..63), 8 values of row
 *   (l % 32) of its block, starting at K = 64 kt + 16 s + 8 (l / 32);
 *   chunks are ordered by K stage kt (64 K), expert e, row block p, step s:
 *   W_packed element ((((kt * E + e) * rows/32 + p) * 4 + s) * 64 + l) * 8 + j
 *   = W[e][row(p, l % 32)][64 kt + 16 s + 8 (l / 32) + j].
 * Pack W1 with gate_up = (act == MOE_SWIGLU), rows = f or 2f, K = d; W2 with
 * gate_up = 0, rows = d, K = f.  Needs rows % 32 == 0 (gate_up: % 64) and
 * K % 64 == 0; W and W_packed 16-byte aligned, not aliased. */
moe_status_t moe_pack_expert_weights(const void *W, int32_t E, int32_t rows, int32_t K, int32_t gate_up,
                                     void *W_packed, void *stream);

/* moe_expert_ffn (bf16) on packed weights, optionally with the dispatch
 * fused in: the same arithmetic and the same output bits as moe_dispatch +
 * moe_expert_ffn on the unpacked weights; the same workspace size
 * (moe_ffn_workspace_size with MOE_BF16) and shape rules.
 *   row_index NULL: X is X_perm (the dispatched rows, slot s = row s; n_x is
 *     ignored).
 *   row_index non-NULL: X is the token matrix [n_x, d] and slot s of expert
 *     e reads X[row_index[s]] (page 2 "The math": X_in = P X, taken by the
 *     GEMM's own row loads instead of a separate gather); pass the routing
 *     map's slot_token.  Entries outside [0, n_x) are clamped into it (the
 *     map never produces them).
 * Y_perm rows are the slots either way; rows >= expert_offset[E] are left
 * untouched. */
moe_status_t moe_expert_ffn_packed(const void *X, int32_t n_x, const int32_t *row_index,
                                   const int32_t *expert_offset, int32_t E, int32_t d, int32_t f, int32_t act,
                                   const void *W1_packed, const void *W2_packed, int64_t M_max, void *Y_perm,
                                   void *ws, size_t ws_bytes, void *stream);

/* moe_expert_ffn_packed for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, kernels and results, without `ws`.  The
 * workspace is a fixed array of MOE_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * and frees nothing.  It serves M_max * f * 2 + MOE_GEMM_WS_BYTES (rounded
 * up to 256) <= MOE_NOALLOC_SCRATCH_BYTES, e.g. M_max * f <= 33 million;
 * larger shapes return MOE_ERR_WORKSPACE (use moe_expert_ffn_packed).  Every
 * call on a GPU uses that GPU's one array, so calls that overlap on one GPU
 * (other streams, other threads) race on it and must be serialised by the
 * caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (64 << 20)
moe_status_t moe_expert_ffn_packed_noalloc(const void *X, int32_t n_x, const int32_t *row_index,
                                           const int32_t *expert_offset, int32_t E, int32_t d, int32_t f,
                                           int32_t act, const void *W1_packed, const void *W2_packed,
                                           int64_t M_max, void *Y_perm, void *stream);

/* The two grouped GEMMs of moe_expert_ffn_packed as separate calls (page 2
 * "The math": Y[e] = Expert_e(X_in[e]); the expert is an up projection with
 * its activation, then a down projection), for a caller that keeps the
 * hidden activation or runs the projections one at a time:
 *   moe_expert_up_packed:   H [M_max, f] = act(X_in W1_e^T) per expert, the
 *     rows of X taken as in moe_expert_ffn_packed (through row_index when
 *     given), fp32 accumulation, H rounded once to bf16;
 *   moe_expert_down_packed: Y_perm [M_max, d] = H W2_e^T per expert.
 * Rows of H / Y_perm at or past expert_offset[E] are left untouched.  The two
 * calls in sequence write the same bits as moe_expert_ffn_packed.  bf16
 * tensors, 16-byte aligned; the same shape rules as moe_expert_ffn_packed; H
 * must not alias X, Y_perm must not alias H.  ws: MOE_GEMM_WS_BYTES of
 * caller-owned device memory, 16-byte aligned (the grouped GEMM's tile
 * counters; overwritten by every call, so calls that may run at the same
 * time need workspaces of their own); a shorter one returns
 * MOE_ERR_WORKSPACE. */
#define MOE_GEMM_WS_BYTES 256
moe_status_t moe_expert_up_packed(const void *X, int32_t n_x, const int32_t *row_index,
                                  const int32_t *expert_offset, int32_t E, int32_t d, int32_t f, int32_t act,
                                  const void *W1_packed, int64_t M_max, void *H, void *ws, size_t ws_bytes,
                                  void *stream);
moe_status_t moe_expert_down_packed(const void *H, const int32_t *expert_offset, int32_t E, int32_t d, int32_t f,
                                    const void *W2_packed, int64_t M_max, void *Y_perm, void *ws, size_t ws_bytes,
                                    void *stream);

/* Combine out = scatter_add(G * Y, I) (page 2 "The math"), the gate applied
 * to the expert output: for every token, out = residual + shared_out + sum
 * of slot_gate[s] * Y_perm[s] over its token_slot list, in list order, fp32
 * accumulation and one rounding to `dtype`.  residual and shared_out [n,d]
 * are optional (NULL = 0).  A token with no kept slot and no shared expert
 * gets its residual back bit for bit (page 1: dropped tokens pass through on
 * the residual stream).  out [n,d]; must not alias the inputs. */
moe_status_t moe_combine(const void *Y_perm, int32_t dtype, const moe_route_map_t *map, int32_t n,
                         int32_t d, const void *residual, const void *shared_out, void *out,
                         void *stream);

/* Balance statistics (page 1 "What each direction guarantees": load-balance
 * loss coefficient 0.01, router z-loss 0.001; page 4 "Pitfalls": monitor
 * per-expert counts, one expert at 80% of traffic means collapse; page 5
 * TL;DR: MaxVio).  Writes stats [MOE_NSTATS] fp32 (layout above) and, when
 * non-NULL, hist [E+1] int32 = number of tokens keeping 0..E experts.
 * Reads logits [n,E] and the map from moe_build_map. */
moe_status_t moe_balance_stats(const float *logits, const moe_route_map_t *map,
                               const moe_route_cfg_t *cfg, float lb_coef, float z_coef, float *stats,
                               int32_t *hist, void *ws, size_t ws_bytes, void *stream);

/* Auxiliary-loss-free balancing (page 5 strategy 4: once per step, the bias
 * of an over-used expert goes down and that of an under-used one up).  Token
 * choice: bias[e] -= gamma * sign(expert_count[e] - n*k/E), the sign taken
 * exactly in integers (an expert exactly at the mean keeps its bias), one
 * fp32 subtraction per expert, in place on the device.  expert_count [E]
 * int32 is the map's pre-drop count (moe_build_map); bias [E] fp32 is the
 * sel_bias of moe_select; gamma finite. */
moe_status_t moe_update_bias(const int32_t *expert_count, const moe_route_cfg_t *cfg, float gamma,
                             float *bias, void *stream);

/* ---- the backward pass ---------------------------------------------------
 * Gradients of L = <dOut, out> + lb_loss + z_loss for one forward, the
 * routing held fixed: the top-k choice, the capacity drops and the counts
 * are piecewise constant in the logits, so they pass no gradient.  The two
 * auxiliary losses are moe_balance_stats' lb_loss and z_loss with the same
 * coefficients (page 1 "What each direction guarantees" gives them as
 * training losses added to the task loss).  One layer's calls, in order:
 *   moe_combine_backward   dY_perm, d_gate            from dOut
 *   moe_expert_ffn_backward dX_perm, dW1, dW2          from dY_perm
 *   (shared expert: moe_expert_ffn_backward with E = 1, offsets {0, n}, on X
 *    and dOut)
 *   moe_gate_backward      dZ                          from d_gate
 *   moe_router_backward    dX_r = dOut + dZ W_g^T, dW_g, d offset
 *   moe_dispatch_backward  dX = dX_r (+ shared dX) + sum over slots of dX_perm
 * bf16 activations are rounded once per stored tensor, products accumulate
 * in fp32, weight gradients are fp32. */

/* Backward of the combine (page 2 "The math": out = scatter_add(G * Y, I)).
 * For every kept slot s < n_kept with t = slot_token[s]:
 *   dY_perm[s] = slot_gate[s] * dOut[t]        (fp32 product, one rounding)
 *   d_gate[s]  = sum_j dOut[t, j] * Y_perm[s, j]  (fp32, a fixed order)
 * dOut [n,d], Y_perm and dY_perm [M_max,d] in dtype; d_gate [M_max] fp32;
 * rows >= n_kept untouched.  The residual's and the shared expert's
 * gradients are dOut itself.  dY_perm must not alias an input. */
moe_status_t moe_combine_backward(const void *dOut, const void *Y_perm, int32_t dtype, int32_t n, int32_t d,
                                  const moe_route_map_t *map, int64_t M_max, void *dY_perm, float *d_gate,
                                  void *stream);

/* Workspace for moe_expert_ffn_backward: the recomputed pre-activation
 * [M_max, f_rows] in fp32, the activation H [M_max, f] and the gradient of
 * the pre-activation [M_max, f_rows] in dtype (f_rows = f, or 2f for
 * SwiGLU), and the weight gradients' work schedule (8 E + 8 int32, also
 * when M_max = 0).  GELU on bf16 with d and f multiples of 8 keeps the
 * pre-activation in registers (one launch computes it and dH) and leaves
 * its part of the workspace untouched; the size is the same either way. */
moe_status_t moe_ffn_backward_workspace_size(int64_t M_max, int32_t E, int32_t d, int32_t f, int32_t act,
                                             int32_t dtype, size_t *bytes);

/* Backward of the expert FFN (page 2 "The math": Y[e] = Expert_e(X_in[e])),
 * per expert e over rows expert_offset[e] .. expert_offset[e+1]-1:
 *   A = X W1^T (recomputed, kept in fp32), H = act(A), dH = dY W2,
 *   dA = dH * act'(A)  (GELU: exact, x Phi(x); SwiGLU: d gate = dH * up *
 *   silu'(gate), d up = dH * silu(gate), gate columns first),
 *   dX_perm = dA W1, dW1[e] = dA^T X_perm, dW2[e] = dY^T H.
 * X_perm, dY_perm, dX_perm [M_max,d] and W1 [E,f_rows,d], W2 [E,d,f] (the
 * natural layout, not packed) in dtype; dW1 [E,f_rows,d] and dW2 [E,d,f]
 * fp32 (16-byte aligned), zero for experts without rows.  bf16 runs on the
 * matrix cores (16-byte aligned tensors); fp32 on a plain kernel.  Errors: invalid
 * shapes, M_max x d, M_max x f_rows or a weight matrix of 2^29 elements or
 * more (byte offsets into the fp32 gradients stay below 2^31),
 * MOE_ERR_WORKSPACE when ws is short. */
moe_status_t moe_expert_ffn_backward(const void *X_perm, int32_t dtype, const int32_t *expert_offset, int32_t E,
                                     int32_t d, int32_t f, int32_t act, const void *W1, const void *W2,
                                     const void *dY_perm, int64_t M_max, void *dX_perm, float *dW1, float *dW2,
                                     void *ws, size_t ws_bytes, void *stream);

/* Backward of the gates and the auxiliary losses to the logits: dZ [n,E]
 * fp32 at `logits` (the router's fp32 output), from d_gate [M_max] (per
 * slot, moe_combine_backward).  Gate formulas as moe_select computes them:
 * token choice softmax over the k selected logits (norm_topk) or the
 * full-row probability; sigmoid / sqrtsoftplus scores renormalised over the
 * k (norm_topk) or raw; expert choice S[t, e] of the row softmax.  A
 * dropped assignment (assign_slot -1) contributes no gate gradient.  Plus
 * lb_coef E f_e / n on every normalised score p_te (f_e = the share of
 * chosen assignments, a constant) and z_coef (2 / n) lse_t softmax(z_t) for
 * the z-loss.  sel_idx [n,k] (token choice; ignored for expert choice) and
 * the map from the forward; every derivative in fp32. */
moe_status_t moe_gate_backward(const float *logits, const int32_t *sel_idx, const float *d_gate,
                               const moe_route_cfg_t *cfg, const moe_route_map_t *map, float lb_coef,
                               float z_coef, float *dZ, void *stream);

/* Workspace for moe_router_backward. */
moe_status_t moe_router_backward_workspace_size(const moe_route_cfg_t *cfg, int32_t dtype, size_t *bytes);

/* Backward of the router Z = X W_g (+ offset) (page 2 "The math"):
 *   dX [n,d] = base + dZ W_g^T (dtype; base [n,d] in dtype or NULL = 0;
 *     dX NULL: skipped),
 *   dWg [d,E] = X^T dZ (fp32; NULL: skipped),
 *   d_offset [E] = column sums of dZ (fp32; NULL: skipped).
 * dZ is rounded to dtype for the products (bf16 on the matrix cores, fp32
 * accumulation).  dX must not alias X or base. */
moe_status_t moe_router_backward(const void *X, const void *Wg, int32_t dtype, const float *dZ,
                                 const moe_route_cfg_t *cfg, const void *base, void *dX, float *dWg,
                                 float *d_offset, void *ws, size_t ws_bytes, void *stream);

/* Backward of the dispatch (page 2 "The math": X_in = P X, so dX = P^T
 * dX_in): dX[t] = base[t] + base2[t] + sum of dX_perm[s] over token t's
 * kept slots in list order, fp32 accumulation, one rounding to dtype.
 * base, base2 [n,d] optional (NULL = 0); dX [n,d] must not alias an input. */
moe_status_t moe_dispatch_backward(const void *dX_perm, int32_t dtype, const moe_route_map_t *map, int32_t n,
                                   int32_t d, const void *base, const void *base2, void *dX, void *stream);

const char *moe_status_string(moe_status_t status);
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DISPATCH_H */
