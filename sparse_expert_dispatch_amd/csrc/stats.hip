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
// Two kernels.  The row kernel (16 waves, R tokens per wave) adds up each
// block's normalised scores, squared log-sum-exps and experts-per-token
// histogram; the final kernel (one workgroup) reduces the block partials in
// a fixed order, so the floats are reproducible bit for bit.  R = 1 unless
// the final workgroup would then need more than two load rounds (many
// blocks, or many experts: each column takes a thread); R = 4 cuts its
// partial rows fourfold.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kStatRows = 16;   // rows per block at one row per wave (the workspace bound)

// NJ = expert registers per lane (experts e = lane + 64 j, j < NJ); R = rows per wave.
template <int NJ, int R>
__global__ __launch_bounds__(1024) void stats_rows_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ token_offset,
                                                         const int32_t* __restrict__ token_slot,
                                                         int n, int E, int score,
                                                         float* __restrict__ part_P,
                                                         float* __restrict__ part_Z,
                                                         int32_t* __restrict__ part_H) {
#pragma clang fp contract(off)
  __shared__ float sP[16][64 * NJ];
  __shared__ float sZ[16];
  __shared__ int sH[kMaxExperts + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int P2 = next_pow2(E);
  for (int i = threadIdx.x; i <= E; i += 1024) sH[i] = 0;
  const int row0 = blockIdx.x * 16 * R + wave * R;
  // every row's list bounds and logits, loaded before the first wait
  int q0[R], q1[R];
  float z[R][NJ];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    const bool in = row < n;
    q0[r] = in ? token_offset[row] : 0;
    q1[r] = in ? token_offset[row + 1] : 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      z[r][j] = in && e < E ? logits[(size_t)row * E + e] : -__builtin_huge_valf();
    }
  }
  // kept experts of each token: its list entries that are not drops
  int kept[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    kept[r] = 0;
    for (int q = q0[r]; q < q1[r]; q += 64)
      kept[r] += __popcll(__ballot(q + lane < q1[r] && token_slot[q + lane] >= 0));
  }
  float accP[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) accP[j] = 0.f;
  float accZ = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (row0 + r >= n) break;
    float m = z[r][0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) m = fmaxf(m, z[r][j]);
    m = wave_max_f32(m);
    float t[NJ], u[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool valid = lane + 64 * j < E;
      t[j] = valid ? spec_exp(z[r][j] - m) : 0.f;
      u[j] = valid ? (score == 0 ? t[j] : spec_expert_score(z[r][j], score)) : 0.f;
    }
    const float s_exp = row_tree_sum(t, P2);
    const float s_norm = score == 0 ? s_exp : row_tree_sum(u, P2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) accP[j] = accP[j] + u[j] / s_norm;
    const float lse = m + logf(s_exp);
    accZ = accZ + lse * lse;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) sP[wave][lane + 64 * j] = accP[j];
  if (lane == 0) sZ[wave] = accZ;
  __syncthreads();   // sH cleared, rows' sums staged
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (row0 + r < n) atomicAdd(&sH[min(kept[r], E)], 1);
  }
  for (int e = threadIdx.x; e < E; e += 1024) {
    float v = sP[0][e];
    for (int w = 1; w < 16; ++w) v = v + sP[w][e];
    part_P[(size_t)blockIdx.x * E + e] = v;
  }
  if (threadIdx.x == 0) {
    float v = sZ[0];
    for (int w = 1; w < 16; ++w) v = v + sZ[w];
    part_Z[blockIdx.x] = v;
  }
  __syncthreads();   // histogram complete
  for (int i = threadIdx.x; i <= E; i += 1024) part_H[(size_t)blockIdx.x * (E + 1) + i] = sH[i];
}

constexpr int kFinThreads = 1024;
constexpr int kFinRows = 16;   // partial rows per thread and load round

MOE_DEV int pow2_at_least(int x, int lo) {
  int p = lo;
  while (p < x) p <<= 1;
  return p;
}

// One workgroup.  Column c of the partial tables (c < E: score sums and
// histogram bins; c = E: the last bin; c = E + 1: squared log-sum-exps) is
// summed by the G = 1024 / cp thread groups (cp = power of two >= E + 2):
// group g takes rows g, g + G, ..., kFinRows of them per round with every
// load of a round issued before the first add; the group sums are then added
// in group order, which fixes the summation order.  After two barriers one
// wave finishes: sum_e f_e P_e by the halving tree over experts (lanes and
// registers), the top non-empty histogram bin from per-wave ballots.
__global__ __launch_bounds__(kFinThreads) void stats_final_kernel(
    const float* __restrict__ part_P, const float* __restrict__ part_Z,
    const int32_t* __restrict__ part_H, int nblocks, int n, int E, int k, int dir, float lb_coef,
    float z_coef, const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset,
    float* __restrict__ stats, int32_t* __restrict__ hist) {
#pragma clang fp contract(off)
  __shared__ float redF[kFinThreads];
  __shared__ int redH[kFinThreads];
  __shared__ float fp[kMaxExperts];
  __shared__ int wred[kFinThreads / 64][3];
  __shared__ float sZ;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- load phase.  Every load is unconditional from a clamped, in-bounds
  // address into a register of its own (the masking comes after), so a
  // round's loads issue back to back with no wait between them.
  const int cnt_raw = expert_count[min(tid, E - 1)];
  const int off_lo = expert_offset[min(tid, E)];
  const int off_hi = expert_offset[min(tid + 1, E)];
  const int n_kept = expert_offset[E];
  const int cp = pow2_at_least(E + 2, 32), G = kFinThreads / cp;
  const int g = tid / cp, c = tid % cp;
  const int cP = min(c, E - 1), cH = min(c, E);
  float sf = 0.f;
  int sh = 0;
  for (int b0 = g; b0 < nblocks; b0 += G * kFinRows) {
    float vp[kFinRows], vz[kFinRows];
    int vh[kFinRows];
#pragma unroll
    for (int u = 0; u < kFinRows; ++u) {
      const int b = min(b0 + u * G, nblocks - 1);
      vp[u] = part_P[(size_t)b * E + cP];
      vz[u] = part_Z[b];
      vh[u] = part_H[(size_t)b * (E + 1) + cH];
    }
    // bit masks rather than selects: every load has an unconditional use,
    // so none is sunk into a branch behind a wait
#pragma unroll
    for (int u = 0; u < kFinRows; ++u) {
      const bool in = b0 + u * G < nblocks;
      const int mp = -(int)(in && c < E), mz = -(int)(in && c == E + 1), mh = -(int)(in && c <= E);
      sf = sf + __int_as_float((__float_as_int(vp[u]) & mp) | (__float_as_int(vz[u]) & mz));
      sh += vh[u] & mh;
    }
  }
  redF[tid] = sf;
  redH[tid] = sh;
  // ---- integer reductions: chosen total, largest kept load
  int chosen = tid < E ? cnt_raw : 0, maxload = tid < E ? off_hi - off_lo : 0;
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
#pragma unroll
  for (int w = 0; w < kFinThreads / 64; ++w) {
    ch += wred[w][0];
    ml = max(ml, wred[w][1]);
  }
  // ---- column totals in group order (the G reads of a column are independent)
  int hv = 0;
  if (tid <= E) {
#pragma unroll 8
    for (int q = 0; q < G; ++q) hv += redH[q * cp + tid];
    if (hist) hist[tid] = hv;
  }
  if (tid < E) {
    float v = 0.f;
#pragma unroll 8
    for (int q = 0; q < G; ++q) v = v + redF[q * cp + tid];
    // f_e = 0 when nothing was chosen (expert choice with k = 0)
    fp[tid] = ch > 0 ? ((float)cnt_raw / (float)ch) * (v / (float)n) : 0.f;
  }
  if (tid == E + 1) {
    float v = 0.f;
#pragma unroll 8
    for (int q = 0; q < G; ++q) v = v + redF[q * cp + tid];
    sZ = v;
  }
  const uint64_t nz = __ballot(tid <= E && hv > 0);
  if (lane == 0) wred[wave][2] = nz ? wave * 64 + 63 - __clzll(nz) : 0;
  __syncthreads();
  if (wave != 0) return;
  float fr[kMaxExpertRegs];
#pragma unroll
  for (int j = 0; j < kMaxExpertRegs; ++j) fr[j] = lane + 64 * j < E ? fp[lane + 64 * j] : 0.f;
  const float fsum = row_tree_sum(fr, next_pow2(E));
  int mt = lane < kFinThreads / 64 ? wred[lane][2] : 0;
  for (int o = 32; o >= 1; o >>= 1) mt = max(mt, __shfl_xor(mt, o, 64));
  if (lane == 0) {
    const int total = dir == 0 ? n * k : E * k;
    const float mean_load = (float)n_kept / (float)E;
    stats[0] = lb_coef * (float)E * fsum;
    stats[1] = z_coef * (sZ / (float)n);
    stats[2] = mean_load > 0.f ? ((float)ml - mean_load) / mean_load : 0.f;
    stats[3] = n_kept > 0 ? (float)ml / (float)n_kept : 0.f;
    stats[4] = (float)n_kept;
    stats[5] = (float)(total - n_kept);
    stats[6] = (float)hv;
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
  // final-kernel load rounds at one row per wave: partial rows / (thread
  // groups x kFinRows), thread groups = 1024 / (power of two >= E + 2)
  const int nb1 = (n + kStatRows - 1) / kStatRows;
  int cp = 32;
  while (cp < E + 2) cp <<= 1;
  const bool four = (int64_t)nb1 * cp > 2LL * kFinThreads * kFinRows;
  const int nb = four ? (n + 4 * kStatRows - 1) / (4 * kStatRows) : nb1;
  char* w = static_cast<char*>(ws);
  float* part_P = reinterpret_cast<float*>(w);
  float* part_Z = reinterpret_cast<float*>(w + align256((size_t)nb * E * sizeof(float)));
  int32_t* part_H = reinterpret_cast<int32_t*>(w + align256((size_t)nb * E * sizeof(float)) +
                                               align256((size_t)nb * sizeof(float)));
  const auto rows = four ? (E <= 64 ? stats_rows_kernel<1, 4>
                            : E <= 128 ? stats_rows_kernel<2, 4>
                            : E <= 256 ? stats_rows_kernel<4, 4>
                                       : stats_rows_kernel<8, 4>)
                     : (E <= 64 ? stats_rows_kernel<1, 1>
                            : E <= 128 ? stats_rows_kernel<2, 1>
                            : E <= 256 ? stats_rows_kernel<4, 1>
                                       : stats_rows_kernel<8, 1>);
  hipLaunchKernelGGL(rows, dim3(nb), dim3(1024), 0, stream, logits, m.token_offset, m.token_slot, n, E,
                     score, part_P, part_Z, part_H);
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
