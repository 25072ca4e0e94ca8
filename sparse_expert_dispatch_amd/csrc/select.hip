// Selection along the expert axis (token choice) or the token axis (expert
// choice) of the token-expert score matrix.
//
// MoE-routing pages: page 2 "Expert choice routing", sections "Token-choice
// and its load-balance headache" (top-k along each row) and "The transposed
// selection" / "The math" (G, I = TopK(S^T, k) along each column); page 5
// "MoE routing strategies explained", strategies 1 (softmax over the k
// selected scores as mixing weights), 2 (top-1), 4 (sigmoid -- or, for
// DeepSeek-V4, sqrtsoftplus -- scores, bias used only when choosing, mixing
// weights from the raw scores) and 5
// (group-limited routing: keep the best groups, then the top-k inside them).
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------- token choice
// One wave per token; lane l holds experts l + 64 j.  Keys become 64-bit
// composites (order-preserving float bits, then the complemented index) so
// one wave-wide unsigned max per round yields the best remaining expert with
// the lower index winning ties.  Group scores: lane g < n_group scans its
// contiguous group in LDS for the top-m keys.
// NJ = expert registers per lane (experts lane + 64 j, j < NJ): the per-lane
// loops run exactly as many times as the row needs.
template <int NJ>
__global__ __launch_bounds__(256) void select_tc_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ bias, SelectArgs a,
                                                        int32_t* __restrict__ idx_out,
                                                        float* __restrict__ gate_out) {
#pragma clang fp contract(off)
  extern __shared__ float smem[];      // per wave: logits [E], keys [E]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int E = a.E;
  float* sz = smem + wave * 2 * E;
  float* sk = sz + E;
  const int t = blockIdx.x * 4 + wave;
  const bool active = t < a.n;
  const int nj = (E + 63) >> 6;
  const float kNegInf = -__builtin_huge_valf();

  float z[NJ], key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    const bool valid = active && j < nj && e < E;
    z[j] = valid ? logits[(size_t)t * E + e] : 0.f;
    if (a.score == 0) {
      key[j] = z[j];
    } else {
      const float s = spec_expert_score(z[j], a.score);
      key[j] = (bias && valid) ? s + bias[e] : s;
    }
    if (valid) {
      sz[e] = z[j];
      sk[e] = key[j];
    }
  }
  __syncthreads();

  if (a.n_group > 1) {
    const int gsz = E / a.n_group;
    uint64_t gk = 0;
    if (active && lane < a.n_group) {
      float top[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
      for (int i = 0; i < gsz; ++i) {
        float v = sk[lane * gsz + i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < a.group_topm && v > top[q]) {
            const float tmp = top[q];
            top[q] = v;
            v = tmp;
          }
        }
      }
      float gs = top[0];
#pragma unroll
      for (int q = 1; q < 4; ++q)
        if (q < a.group_topm) gs = gs + top[q];
      gk = rank_key(gs, (uint32_t)lane);
    }
    uint64_t keep = 0;
    for (int r = 0; r < a.topk_group; ++r) {
      const uint64_t w = wave_max_u64(gk);
      const uint32_t g = rank_key_index(w);
      if (g < 64) keep |= 1ull << g;
      if ((uint32_t)lane == g) gk = 0;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (j < nj && e < E && !((keep >> (e / gsz)) & 1ull)) key[j] = kNegInf;
    }
  }

  uint64_t ck[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    ck[j] = (active && j < nj && e < E) ? rank_key(key[j], (uint32_t)e) : 0ull;
  }
  int my_sel = 0;   // lane r < k: the rank-r expert
  for (int r = 0; r < a.k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) best = ck[j] > best ? ck[j] : best;
    const uint64_t w = wave_max_u64(best);
    const int e = (int)rank_key_index(w);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (lane + 64 * j == e) ck[j] = 0ull;
    if (lane == r) my_sel = e;
  }
  if (!active) return;

  // Gates.
  float gate = 0.f;
  if (a.score == 0) {
    if (a.norm_topk) {
      // softmax over the k selected logits, shifted by the top one; summed
      // left to right in rank order
      const float ztop = sz[__shfl(my_sel, 0, 64)];
      float s = 0.f;
      for (int j = 0; j < a.k; ++j) s = s + spec_exp(sz[__shfl(my_sel, j, 64)] - ztop);
      gate = spec_exp(sz[my_sel] - ztop) / s;
    } else {
      // the full-row softmax probability
      float m = kNegInf;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (j < nj && lane + 64 * j < E) m = fmaxf(m, z[j]);
      m = wave_max_f32(m);
      float tt[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        tt[j] = (j < nj && lane + 64 * j < E) ? spec_exp(z[j] - m) : 0.f;
      const float s = row_tree_sum(tt, next_pow2(E));
      gate = spec_exp(sz[my_sel] - m) / s;
    }
  } else {
    const float mine = spec_expert_score(sz[my_sel], a.score);
    if (a.norm_topk) {
      float s = 0.f;
      for (int j = 0; j < a.k; ++j) s = s + spec_expert_score(sz[__shfl(my_sel, j, 64)], a.score);
      gate = mine / s;
    } else {
      gate = mine;
    }
  }
  if (lane < a.k) {
    idx_out[(size_t)t * a.k + lane] = my_sel;
    gate_out[(size_t)t * a.k + lane] = gate;
  }
}

hipError_t launch_select_tc(const float* logits, const float* bias, const SelectArgs& a, int32_t* idx,
                            float* gate, hipStream_t stream) {
  const size_t lds = (size_t)4 * 2 * a.E * sizeof(float);
  const int nj = (a.E + 63) / 64;
  const auto kern = nj <= 1 ? select_tc_kernel<1> : nj <= 2 ? select_tc_kernel<2>
                  : nj <= 4 ? select_tc_kernel<4> : select_tc_kernel<8>;
  hipLaunchKernelGGL(kern, dim3((a.n + 3) / 4), dim3(256), lds, stream, logits, bias, a, idx, gate);
  return hipGetLastError();
}

// ---------------------------------------------------------------- expert choice
// One workgroup (16 waves) per expert.  The column S[:, e] (contiguous in
// S^T) becomes order-preserving uint32 keys, staged in LDS when they fit.  An
// MSB-first radix select (4 passes of 8 bits, LDS histograms) finds the
// exact k-th largest key T and how many keys equal to T must be taken; a
// block-wide scan in token order then emits every key > T and the first
// `take` keys == T, which yields the lowest-index tie-break and ascending
// token order in one pass.

constexpr int kEcThreads = 1024;
constexpr int kEcLdsKeys = 32768;   // keys staged in LDS up to this n

template <bool kLds>
__global__ __launch_bounds__(kEcThreads) void select_ec_kernel(const float* __restrict__ scores_t,
                                                               int n, int k, int32_t* __restrict__ I,
                                                               float* __restrict__ G) {
  extern __shared__ uint32_t skeys[];
  __shared__ int hist[256];
  __shared__ int wave_tot[kEcThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int e = blockIdx.x;
  const float* col = scores_t + (size_t)e * n;

  if (kLds) {
    for (int i = tid; i < n; i += kEcThreads) skeys[i] = order_key(col[i]);
  }
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kEcThreads) {
      const uint32_t key = kLds ? skeys[i] : order_key(col[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      int c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[255 - 4 * lane - q];
      const int local = c[0] + c[1] + c[2] + c[3];
      const int incl = wave_inclusive_scan_i32(local);
      const uint64_t hit = __ballot(incl >= remaining);
      const int first = __ffsll((unsigned long long)hit) - 1;
      if (lane == first) {
        int cum = incl - local;
        int D = 255 - 4 * lane - 3, rem = remaining - cum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + c[q] >= remaining) {
            D = 255 - 4 * lane - q;
            rem = remaining - cum;
            break;
          }
          cum += c[q];
        }
        s_prefix = prefix | ((uint32_t)D << shift);
        s_remaining = rem;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 0xFFu << shift;
  }
  const uint32_t T = prefix;
  const int take = remaining;           // keys equal to T to keep, lowest index first

  int run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += kEcThreads) {
    const int i = base + tid;
    uint32_t key = 0;
    if (i < n) key = kLds ? skeys[i] : order_key(col[i]);
    const int gt = (i < n && key > T) ? 1 : 0;
    const int eq = (i < n && key == T) ? 1 : 0;
    const int packed = gt | (eq << 16);
    const int incl = wave_inclusive_scan_i32(packed);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      const int v = lane < kEcThreads / 64 ? wave_tot[lane] : 0;
      const int sc = wave_inclusive_scan_i32(v);
      if (lane < kEcThreads / 64) wave_tot[lane] = sc - v;      // exclusive
      if (lane == kEcThreads / 64 - 1) s_prefix = (uint32_t)sc;  // chunk total
    }
    __syncthreads();
    const int excl = wave_tot[wave] + incl - packed;
    const int gt_before = run_gt + (excl & 0xFFFF);
    const int eq_before = run_eq + (excl >> 16);
    const bool sel = gt || (eq && eq_before < take);
    if (sel) {
      const int pos = gt_before + min(eq_before, take);
      I[(size_t)e * k + pos] = i;
      G[(size_t)e * k + pos] = col[i];
    }
    const uint32_t tot = s_prefix;
    run_gt += (int)(tot & 0xFFFFu);
    run_eq += (int)(tot >> 16);
    __syncthreads();
  }
}

size_t select_ec_workspace_bytes(int n, int E) { return (size_t)n * E * sizeof(float); }

hipError_t launch_select_ec(const float* logits, const float* scores_t, int n, int E, int k,
                            int32_t* I, float* G, void* ws, hipStream_t stream) {
  if (!scores_t) {
    float* st = static_cast<float*>(ws);
    hipError_t err = launch_router_finalize(logits, 1, n, E, nullptr, nullptr, 0.f, 0, nullptr, nullptr, st,
                                            stream);
    if (err != hipSuccess) return err;
    scores_t = st;
  }
  if (n <= kEcLdsKeys) {
    const size_t lds = (size_t)n * sizeof(uint32_t);
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_ec_kernel<true>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kEcLdsKeys * (int)sizeof(uint32_t));
      if (err != hipSuccess) return err;
      attr_set = true;
    }
    hipLaunchKernelGGL(select_ec_kernel<true>, dim3(E), dim3(kEcThreads), lds, stream, scores_t, n, k,
                       I, G);
  } else {
    hipLaunchKernelGGL(select_ec_kernel<false>, dim3(E), dim3(kEcThreads), 0, stream, scores_t, n, k,
                       I, G);
  }
  return hipGetLastError();
}

}  // namespace moe
