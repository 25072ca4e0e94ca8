// Routing-balance statistics.
//
// MoE-routing pages: page 1 "Token choice vs expert choice routing", section
// "What each direction guarantees" (load-balancing loss at 0.01 and router
// z-loss at 0.001; a balanced router gives every expert the same share);
// page 4 "How MoE routing strategies ...", section "Pitfalls" (watch
// per-expert token counts; one expert with 80% of the traffic means the
// router collapsed); page 5 "MoE routing strategies explained", TL;DR
// (MaxVio).  The pages name these quantities without formulas; the library
// computes
//   lb_loss = lb_coef * E * sum_e f_e * P_e,  f_e = chosen_e / sum chosen,
//             P_e = mean over tokens of the normalised score (softmax
//             probability, or sigmoid / row sum of sigmoids),
//   z_loss  = z_coef * mean_t (logsumexp_e z_te)^2,
//   max_vio = (max_e load_e - mean load) / mean load,  load = kept rows,
// plus kept / dropped counts and the experts-per-token histogram.
//
// Deterministic: per-block partial sums in a fixed order, then one
// workgroup reduces them in block order; integers use order-free atomics.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kStatRows = 64;   // rows per block (16 per wave)

__global__ __launch_bounds__(256) void stats_rows_kernel(const float* __restrict__ logits, int n,
                                                         int E, int score, float* __restrict__ part_P,
                                                         float* __restrict__ part_Z) {
#pragma clang fp contract(off)
  __shared__ float sP[4][kMaxExperts];
  __shared__ float sZ[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nj = (E + 63) >> 6;
  const int P2 = next_pow2(E);
  float accP[kMaxExpertRegs];
#pragma unroll
  for (int j = 0; j < kMaxExpertRegs; ++j) accP[j] = 0.f;
  float accZ = 0.f;
  for (int r = 0; r < kStatRows / 4; ++r) {
    const int row = blockIdx.x * kStatRows + wave * (kStatRows / 4) + r;
    if (row >= n) break;
    float z[kMaxExpertRegs];
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) {
      const int e = lane + 64 * j;
      z[j] = (j < nj && e < E) ? logits[(size_t)row * E + e] : 0.f;
      if (j < nj && e < E) m = fmaxf(m, z[j]);
    }
    m = wave_max_f32(m);
    float t[kMaxExpertRegs], u[kMaxExpertRegs];
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) {
      const bool valid = j < nj && lane + 64 * j < E;
      t[j] = valid ? spec_exp(z[j] - m) : 0.f;
      u[j] = valid ? (score == 0 ? t[j] : spec_sigmoid(z[j])) : 0.f;
    }
    const float s_exp = row_tree_sum(t, P2);
    const float s_norm = score == 0 ? s_exp : row_tree_sum(u, P2);
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) accP[j] = accP[j] + u[j] / s_norm;
    const float lse = m + logf(s_exp);
    accZ = accZ + lse * lse;
  }
#pragma unroll
  for (int j = 0; j < kMaxExpertRegs; ++j) {
    const int e = lane + 64 * j;
    if (j < nj && e < E) sP[wave][e] = accP[j];
  }
  if (lane == 0) sZ[wave] = accZ;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    part_P[(size_t)blockIdx.x * E + e] = ((sP[0][e] + sP[1][e]) + sP[2][e]) + sP[3][e];
  if (threadIdx.x == 0) part_Z[blockIdx.x] = ((sZ[0] + sZ[1]) + sZ[2]) + sZ[3];
}

constexpr int kFinThreads = 1024;

__global__ __launch_bounds__(kFinThreads) void stats_final_kernel(
    const float* __restrict__ part_P, const float* __restrict__ part_Z, int nblocks, int n, int E,
    int k, int dir, float lb_coef, float z_coef, const int32_t* __restrict__ expert_count,
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ token_offset,
    float* __restrict__ stats, int32_t* __restrict__ hist) {
#pragma clang fp contract(off)
  __shared__ float red[kFinThreads];
  __shared__ int ired[kFinThreads];
  __shared__ int shist[kMaxExperts + 1];
  const int tid = threadIdx.x;

  // total chosen assignments (exact integer)
  ired[tid] = tid < E ? expert_count[tid] : 0;
  __syncthreads();
  for (int s = kFinThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) ired[tid] += ired[tid + s];
    __syncthreads();
  }
  const int chosen_total = ired[0];
  __syncthreads();

  // f_e * P_e, reduced by a fixed tree over experts
  float fp = 0.f;
  if (tid < E) {
    float pe = 0.f;
    for (int b = 0; b < nblocks; ++b) pe = pe + part_P[(size_t)b * E + tid];
    pe = pe / (float)n;
    const float fe = (float)expert_count[tid] / (float)chosen_total;
    fp = fe * pe;
  }
  red[tid] = fp;
  __syncthreads();
  for (int s = kFinThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) red[tid] = red[tid] + red[tid + s];
    __syncthreads();
  }
  const float sum_fp = red[0];
  __syncthreads();

  // z-loss partials, fixed tree over blocks (nblocks may exceed the thread count)
  float zp = 0.f;
  for (int b = tid; b < nblocks; b += kFinThreads) zp = zp + part_Z[b];
  red[tid] = zp;
  __syncthreads();
  for (int s = kFinThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) red[tid] = red[tid] + red[tid + s];
    __syncthreads();
  }
  const float sum_z = red[0];
  __syncthreads();

  // maximum kept load
  ired[tid] = tid < E ? expert_offset[tid + 1] - expert_offset[tid] : 0;
  __syncthreads();
  for (int s = kFinThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) ired[tid] = max(ired[tid], ired[tid + s]);
    __syncthreads();
  }
  const int max_load = ired[0];
  __syncthreads();

  // experts-per-token histogram and its maximum
  for (int i = tid; i <= E; i += kFinThreads) shist[i] = 0;
  __syncthreads();
  int my_max = 0;
  for (int t = tid; t < n; t += kFinThreads) {
    const int c = token_offset[t + 1] - token_offset[t];
    atomicAdd(&shist[min(c, E)], 1);
    my_max = max(my_max, c);
  }
  ired[tid] = my_max;
  __syncthreads();
  for (int s = kFinThreads / 2; s >= 1; s >>= 1) {
    if (tid < s) ired[tid] = max(ired[tid], ired[tid + s]);
    __syncthreads();
  }
  const int max_per_token = ired[0];
  if (hist)
    for (int i = tid; i <= E; i += kFinThreads) hist[i] = shist[i];

  if (tid == 0) {
    const int n_kept = expert_offset[E];
    const int total = dir == 0 ? n * k : E * k;
    const float mean_load = (float)n_kept / (float)E;
    stats[0] = lb_coef * (float)E * sum_fp;
    stats[1] = z_coef * (sum_z / (float)n);
    stats[2] = mean_load > 0.f ? ((float)max_load - mean_load) / mean_load : 0.f;
    stats[3] = n_kept > 0 ? (float)max_load / (float)n_kept : 0.f;
    stats[4] = (float)n_kept;
    stats[5] = (float)(total - n_kept);
    stats[6] = (float)shist[0];
    stats[7] = (float)max_per_token;
  }
}

size_t stats_workspace_bytes(int n, int E) {
  const size_t nb = (size_t)(n + kStatRows - 1) / kStatRows;
  return nb * E * sizeof(float) + nb * sizeof(float);
}

hipError_t launch_balance_stats(const float* logits, const MapPtrs& m, int n, int E, int k, int dir,
                                int score, float lb_coef, float z_coef, float* stats, int32_t* hist,
                                void* ws, hipStream_t stream) {
  const int nb = (n + kStatRows - 1) / kStatRows;
  float* part_P = static_cast<float*>(ws);
  float* part_Z = part_P + (size_t)nb * E;
  hipLaunchKernelGGL(stats_rows_kernel, dim3(nb), dim3(256), 0, stream, logits, n, E, score, part_P,
                     part_Z);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kFinThreads), 0, stream, part_P, part_Z, nb, n,
                     E, k, dir, lb_coef, z_coef, m.expert_count, m.expert_offset, m.token_offset,
                     stats, hist);
  return hipGetLastError();
}

}  // namespace moe
