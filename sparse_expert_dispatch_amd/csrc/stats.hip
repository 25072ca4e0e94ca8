// Routing-balance statistics.
//
// MoE-routing pages: page 1 "Token choice vs expert choice routing", section
// "What each direction guarantees" (coefficients 0.01 for the load-balancing
// loss and 0.001 for the z-loss; a balanced router gives every expert the
// same share);
// page 4 "How MoE routing strategies ...", section "Pitfalls" (watch
// per-expert token counts; one expert with 80% of the traffic means the
// router collapsed); page 5 "MoE routing strategies explained", TL;DR
// (MaxVio).  The pages name these quantities without formulas; the library
// computes
//   lb_loss = lb_coef * E * sum_e f_e * P_e,  f_e = chosen_e / sum chosen,
//             P_e = mean over tokens of the normalised score (softmax
//             probability, or sigmoid / sqrtsoftplus score over its row sum),
//   z_loss  = z_coef * mean_t (logsumexp_e z_te)^2,
//   max_vio = (max_e load_e - mean load) / mean load,  load = kept rows,
// plus kept / dropped counts and the experts-per-token histogram.
//
// Two kernels.  The row kernel (16 tokens per workgroup, one per wave) adds up
// each block's normalised scores, squared log-sum-exps and experts-per-token
// histogram; the final kernel (one workgroup) reduces the block partials in
// a fixed order, so the floats are reproducible bit for bit.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kStatRows = 16;   // rows per block, one per wave

__global__ __launch_bounds__(1024) void stats_rows_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ token_offset,
                                                         const int32_t* __restrict__ token_slot,
                                                         int n, int E, int score,
                                                         float* __restrict__ part_P,
                                                         float* __restrict__ part_Z,
                                                         int32_t* __restrict__ part_H) {
#pragma clang fp contract(off)
  __shared__ float sP[kStatRows][kMaxExperts];
  __shared__ float sZ[kStatRows];
  __shared__ int sH[kMaxExperts + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nj = (E + 63) >> 6;
  const int P2 = next_pow2(E);
  for (int i = threadIdx.x; i <= E; i += 1024) sH[i] = 0;
  __syncthreads();
  float accP[kMaxExpertRegs];
#pragma unroll
  for (int j = 0; j < kMaxExpertRegs; ++j) accP[j] = 0.f;
  float accZ = 0.f;
  {
    const int row = blockIdx.x * kStatRows + wave;
    if (row >= n) goto done;
    float z[kMaxExpertRegs];
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) {
      const int e = lane + 64 * j;
      z[j] = (j < nj && e < E) ? logits[(size_t)row * E + e] : 0.f;
      if (j < nj && e < E) m = fmaxf(m, z[j]);
    }
    // kept experts of this token: its list entries that are not drops
    const int q0 = token_offset[row], q1 = token_offset[row + 1];
    int kept = 0;
    for (int q = q0; q < q1; q += 64)
      kept += __popcll(__ballot(q + lane < q1 && token_slot[q + lane] >= 0));
    if (lane == 0) atomicAdd(&sH[min(kept, E)], 1);
    m = wave_max_f32(m);
    float t[kMaxExpertRegs], u[kMaxExpertRegs];
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) {
      const bool valid = j < nj && lane + 64 * j < E;
      t[j] = valid ? spec_exp(z[j] - m) : 0.f;
      u[j] = valid ? (score == 0 ? t[j] : spec_expert_score(z[j], score)) : 0.f;
    }
    const float s_exp = row_tree_sum(t, P2);
    const float s_norm = score == 0 ? s_exp : row_tree_sum(u, P2);
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) accP[j] = accP[j] + u[j] / s_norm;
    const float lse = m + logf(s_exp);
    accZ = accZ + lse * lse;
  }
done:
#pragma unroll
  for (int j = 0; j < kMaxExpertRegs; ++j) {
    const int e = lane + 64 * j;
    if (j < nj && e < E) sP[wave][e] = accP[j];
  }
  if (lane == 0) sZ[wave] = accZ;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) {
    float v = sP[0][e];
    for (int w = 1; w < kStatRows; ++w) v = v + sP[w][e];
    part_P[(size_t)blockIdx.x * E + e] = v;
  }
  for (int i = threadIdx.x; i <= E; i += 1024) part_H[(size_t)blockIdx.x * (E + 1) + i] = sH[i];
  if (threadIdx.x == 0) {
    float v = sZ[0];
    for (int w = 1; w < kStatRows; ++w) v = v + sZ[w];
    part_Z[blockIdx.x] = v;
  }
}

constexpr int kFinThreads = 1024;

MOE_DEV int pow2_at_least(int x, int lo) {
  int p = lo;
  while (p < x) p <<= 1;
  return p;
}

// One workgroup.  Every global value it needs is loaded in one phase (no
// barrier in between, so the loads are all in flight together): thread group
// g of the partial tables sums rows g, g + G, ... of its column; the group
// sums are then added in group order, which fixes the summation order.
__global__ __launch_bounds__(kFinThreads) void stats_final_kernel(
    const float* __restrict__ part_P, const float* __restrict__ part_Z,
    const int32_t* __restrict__ part_H, int nblocks, int n, int E, int k, int dir, float lb_coef,
    float z_coef, const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset,
    float* __restrict__ stats, int32_t* __restrict__ hist) {
#pragma clang fp contract(off)
  __shared__ float redP[kFinThreads];
  __shared__ float redZ[kFinThreads];
  __shared__ int redH[kFinThreads];
  __shared__ float fp[kMaxExperts];
  __shared__ int sH[kMaxExperts + 1];
  __shared__ int wred[kFinThreads / 64][2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- load phase
  const int cpP = pow2_at_least(E, 32), gP = kFinThreads / cpP;
  const int cpH = pow2_at_least(E + 1, 32), gH = kFinThreads / cpH;
  float sp = 0.f, sz = 0.f;
  int sh = 0;
  {
    const int g = tid / cpP, c = tid % cpP;
    if (c < E) {
#pragma unroll 16
      for (int b = g; b < nblocks; b += gP) sp = sp + part_P[(size_t)b * E + c];
    }
  }
  {
    const int g = tid / cpH, c = tid % cpH;
    if (c <= E) {
#pragma unroll 16
      for (int b = g; b < nblocks; b += gH) sh += part_H[(size_t)b * (E + 1) + c];
    }
  }
#pragma unroll 4
  for (int b = tid; b < nblocks; b += kFinThreads) sz = sz + part_Z[b];
  const int cnt = tid < E ? expert_count[tid] : 0;
  const int load = tid < E ? expert_offset[tid + 1] - expert_offset[tid] : 0;
  const int n_kept = expert_offset[E];
  redP[tid] = sp;
  redH[tid] = sh;
  redZ[tid] = sz;
  // ---- integer reductions: chosen total, largest kept load
  int chosen = cnt, maxload = load;
  for (int o = 32; o >= 1; o >>= 1) {
    chosen += __shfl_xor(chosen, o, 64);
    maxload = max(maxload, __shfl_xor(maxload, o, 64));
  }
  if (lane == 0) {
    wred[wave][0] = chosen;
    wred[wave][1] = maxload;
  }
  __syncthreads();
  int ch = 0, ml = 0;
  for (int w = 0; w < kFinThreads / 64; ++w) {
    ch += wred[w][0];
    ml = max(ml, wred[w][1]);
  }
  if (tid <= E) {
    int v = 0;
    for (int q = 0; q < gH; ++q) v += redH[q * cpH + tid];
    sH[tid] = v;
    if (hist) hist[tid] = v;
  }
  if (tid < E) {
    float v = 0.f;
    for (int q = 0; q < gP; ++q) v = v + redP[q * cpP + tid];
    // f_e = 0 when nothing was chosen (expert choice with k = 0)
    fp[tid] = ch > 0 ? ((float)cnt / (float)ch) * (v / (float)n) : 0.f;
  }
  // z partials: a halving tree over the 1024 thread sums
  for (int s = kFinThreads / 2; s >= 1; s >>= 1) {
    __syncthreads();
    if (tid < s) redZ[tid] = redZ[tid] + redZ[tid + s];
  }
  // sum_e f_e P_e by a halving tree over experts
  const int P = next_pow2(E);
  for (int s = P >> 1; s >= 1; s >>= 1) {
    __syncthreads();
    if (tid < s) fp[tid] = fp[tid] + (tid + s < E ? fp[tid + s] : 0.f);
  }
  __syncthreads();
  if (tid == 0) {
    int mt = 0;
    for (int i = E; i >= 0; --i)
      if (sH[i] > 0) {
        mt = i;
        break;
      }
    const int total = dir == 0 ? n * k : E * k;
    const float mean_load = (float)n_kept / (float)E;
    stats[0] = lb_coef * (float)E * fp[0];
    stats[1] = z_coef * (redZ[0] / (float)n);
    stats[2] = mean_load > 0.f ? ((float)ml - mean_load) / mean_load : 0.f;
    stats[3] = n_kept > 0 ? (float)ml / (float)n_kept : 0.f;
    stats[4] = (float)n_kept;
    stats[5] = (float)(total - n_kept);
    stats[6] = (float)sH[0];
    stats[7] = (float)mt;
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t stats_workspace_bytes(int n, int E) {
  const size_t nb = (size_t)(n + kStatRows - 1) / kStatRows;
  return align256(nb * E * sizeof(float)) + align256(nb * sizeof(float)) +
         align256(nb * (E + 1) * sizeof(int32_t));
}

hipError_t launch_balance_stats(const float* logits, const MapPtrs& m, int n, int E, int k, int dir,
                                int score, float lb_coef, float z_coef, float* stats, int32_t* hist,
                                void* ws, hipStream_t stream) {
  const int nb = (n + kStatRows - 1) / kStatRows;
  char* w = static_cast<char*>(ws);
  float* part_P = reinterpret_cast<float*>(w);
  float* part_Z = reinterpret_cast<float*>(w + align256((size_t)nb * E * sizeof(float)));
  int32_t* part_H = reinterpret_cast<int32_t*>(w + align256((size_t)nb * E * sizeof(float)) +
                                               align256((size_t)nb * sizeof(float)));
  hipLaunchKernelGGL(stats_rows_kernel, dim3(nb), dim3(1024), 0, stream, logits, m.token_offset,
                     m.token_slot, n, E, score, part_P, part_Z, part_H);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kFinThreads), 0, stream, part_P, part_Z, part_H,
                     nb, n, E, k, dir, lb_coef, z_coef, m.expert_count, m.expert_offset, stats, hist);
  return hipGetLastError();
}

// Loss-free balancing step (page 5 "MoE routing strategies explained",
// strategy 4: once per step, the bias of an over-used expert goes down and
// that of an under-used one up): bias[e] -= gamma * sign(count[e] - n k / E), the sign
// from the exact integer comparison count[e] * E vs n * k, so an expert
// exactly at the mean keeps its bias.  One thread per expert.
__global__ __launch_bounds__(256) void update_bias_kernel(const int32_t* __restrict__ count, int E,
                                                          int64_t nk, float gamma, float* __restrict__ bias) {
#pragma clang fp contract(off)
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t diff = (int64_t)count[e] * E - nk;
  const float sgn = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
  bias[e] = bias[e] - gamma * sgn;
}

hipError_t launch_update_bias(const int32_t* expert_count, int n, int E, int k, float gamma, float* bias,
                              hipStream_t stream) {
  hipLaunchKernelGGL(update_bias_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, expert_count, E,
                     (int64_t)n * k, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
