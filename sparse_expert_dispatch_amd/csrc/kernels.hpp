// Internal launch interface between the C ABI layer (api.cpp) and the HIP
// kernels.  Launchers enqueue on `stream` and return hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 512;      // experts per layer
constexpr int kMaxExpertRegs = kMaxExperts / 64;

#ifdef __HIPCC__
// Halving-stride tree sum of a zero-padded power-of-two row of length P
// held as lane l, register j -> element l + 64 j.  Passes with a stride of
// 64 s elements are in-register (j += s); the last six are across lanes.
// Returns the sum in every lane; `row` is not modified.
template <int R>
__device__ __forceinline__ float row_tree_sum(const float (&row)[R], int P) {
#pragma clang fp contract(off)
  float t[R];
#pragma unroll
  for (int j = 0; j < R; ++j) t[j] = row[j];
#pragma unroll
  for (int s = R / 2; s >= 1; s >>= 1) {
    if (s < (P >> 6)) {
#pragma unroll
      for (int j = 0; j < s; ++j) t[j] = t[j] + t[j + s];
    }
  }
  float v = t[0];
  const int Pw = P < 64 ? P : 64;
  for (int s = Pw >> 1; s >= 1; s >>= 1) v = v + __shfl_down(v, s, 64);
  return __shfl(v, 0, 64);
}
#endif

// router.hip
size_t router_workspace_bytes(int n, int d, int E, int dtype, int score);
hipError_t launch_router(const void* X, const void* Wg, int dtype, const float* offset,
                         const float* noise, float noise_std, int n, int d, int E, int score,
                         float* logits, float* scores, float* scores_t, void* ws, hipStream_t stream);

// Scores (and/or their transpose) from finished logits: the router's
// epilogue on its own; `logits` may be NULL.
hipError_t launch_router_finalize(const float* partial, int nsplit, int n, int E, const float* offset,
                                  const float* noise, float noise_std, int score, float* logits,
                                  float* scores, float* scores_t, hipStream_t stream);

// select.hip
struct SelectArgs {
  int n, E, k, score, n_group, topk_group, group_topm, norm_topk;
};
hipError_t launch_select_tc(const float* logits, const float* bias, const SelectArgs& a, int32_t* idx,
                            float* gate, hipStream_t stream);
size_t select_ec_workspace_bytes(int n, int E);
hipError_t launch_select_ec(const float* logits, const float* scores_t, int n, int E, int k,
                            int32_t* I, float* G, void* ws, hipStream_t stream);

// route_map.hip
struct MapPtrs {
  int32_t* expert_count;
  int32_t* expert_offset;
  int32_t* slot_token;
  float* slot_gate;
  int32_t* assign_slot;
  int32_t* token_offset;
  int32_t* token_slot;
  int32_t* n_kept;
};
size_t map_workspace_bytes(int dir, int n, int E, int k);
hipError_t launch_build_map_tc(const int32_t* idx, const float* gate, int n, int E, int k,
                               int capacity, int rank_major, const MapPtrs& m, void* ws,
                               hipStream_t stream);
hipError_t launch_build_map_ec(const int32_t* I, const float* G, int n, int E, int k,
                               const MapPtrs& m, void* ws, hipStream_t stream);

// permute.hip
hipError_t launch_dispatch(const void* X, int elem_bytes, int n, int d, const int32_t* slot_token,
                           const int32_t* n_kept, int64_t M_max, void* X_perm, hipStream_t stream);
hipError_t launch_combine(const void* Y, int dtype, const int32_t* token_offset,
                          const int32_t* token_slot, const float* slot_gate, int n, int d,
                          const void* residual, const void* shared, void* out, hipStream_t stream);

// grouped_gemm.hip
size_t ffn_workspace_bytes(int64_t M_max, int E, int d, int f, int act, int dtype);
// row_index (bf16 only): the up GEMM's A row of slot s is X_perm[row_index[s]]
// (X_perm then has n_x rows); nullptr: row s.
hipError_t launch_expert_ffn(const void* X_perm, const int32_t* row_index, int n_x, int dtype,
                             const int32_t* expert_offset, int E, int d, int f, int act, const void* W1,
                             const void* W2, int64_t M_max, void* Y_perm, void* ws, bool packed,
                             hipStream_t stream);
hipError_t launch_pack_weights(const void* W, int E, int R, int K, int gate_up, void* P, hipStream_t stream);
// One bf16 grouped GEMM of the FFN: stage 1 the up projection (A = token rows
// through row_index when given, W = W1, C = H [M_max, f]), stage 2 the down
// projection (A = H, W = W2, C = Y_perm).  ws: kGemmWsBytes of device memory
// (tile counters of the weight-streaming kernel).
constexpr size_t kGemmWsBytes = 256;
hipError_t launch_expert_gemm(int stage, const void* A, const int32_t* row_index, int n_a,
                              const int32_t* expert_offset, int E, int d, int f, int act, const void* W,
                              int64_t M_max, void* C, bool packed, void* ws, hipStream_t stream);

// The backward's pre-activation recompute: C [rows, N] fp32 = A W^T per
// expert (A [rows, K] bf16, W [E, N, K] bf16 natural layout), K % 64 == 0.
hipError_t launch_rows_gemm_f32(const void* A, const int32_t* expert_offset, int E, const void* W, int N, int K,
                                int64_t M_max, float* C, hipStream_t stream);

// The backward's dX: C [rows, N] bf16 = A W per expert with W [E, K, N]
// bf16 (K-major), A [rows, K] bf16; K % 64 == 0, N % 8 == 0.
hipError_t launch_rows_gemm_kmajor(const void* A, const int32_t* expert_offset, int E, const void* W, int N, int K,
                                   int64_t M_max, void* C, hipStream_t stream);

// noalloc.hip: the device address of this library's fixed workspace array
// on the current device (MOE_NOALLOC_SCRATCH_BYTES), looked up once per
// device.
hipError_t noalloc_scratch(void** ptr);

// backward.hip
hipError_t launch_combine_backward(const void* dout, const void* Y, int dtype, int d, const int32_t* slot_token,
                                   const float* slot_gate, const int32_t* n_kept, int64_t M_max, void* dY,
                                   float* d_gate, hipStream_t stream);
hipError_t launch_gate_backward(const float* logits, const int32_t* sel_idx, const float* d_gate,
                                const MapPtrs& m, int n, int E, int k, int dir, int score, int norm_topk,
                                float lb_coef, float z_coef, float* dZ, hipStream_t stream);
size_t ffn_backward_workspace_bytes(int64_t M_max, int E, int d, int f, int act, int dtype);
hipError_t launch_expert_ffn_backward(const void* X_perm, int dtype, const int32_t* expert_offset, int E, int d,
                                      int f, int act, const void* W1, const void* W2, const void* dY_perm,
                                      int64_t M_max, void* dX_perm, float* dW1, float* dW2, void* ws,
                                      hipStream_t stream);
size_t router_backward_workspace_bytes(int n, int d, int E, int dtype);
hipError_t launch_router_backward(const void* X, const void* Wg, int dtype, const float* dZ, int n, int d, int E,
                                  const void* base, void* dX, float* dWg, float* d_offset, void* ws,
                                  hipStream_t stream);

// stats.hip
size_t stats_workspace_bytes(int n, int E);
hipError_t launch_balance_stats(const float* logits, const MapPtrs& m, int n, int E, int k, int dir,
                                int score, float lb_coef, float z_coef, float* stats, int32_t* hist,
                                void* ws, hipStream_t stream);
hipError_t launch_update_bias(const int32_t* expert_count, int n, int E, int k, float gamma, float* bias,
                              hipStream_t stream);

}  // namespace moe
