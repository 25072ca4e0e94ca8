// Backward pass of the MoE layer: gradients of L = <dOut, out> + lb_loss +
// z_loss with the routing (choice, drops, counts) held fixed.
//
// MoE-routing pages: page 2 "Expert choice routing", section "The math"
// (X_in = P X, Y = Expert(X_in), out = scatter_add(G * Y, I): the backward
// runs these maps in reverse); page 1 "Token choice vs expert choice
// routing", section "What each direction guarantees" (the auxiliary loss
// coefficients); page 5 "MoE routing strategies explained", strategies 1
// and 4 (softmax and sigmoid gates).
//
// Kernels:
// * combine backward: one wave per kept slot: dY = gate * dOut[token] and
//   d_gate = <dOut[token], Y> (fixed-order fp32 dot product);
// * gate backward: one wave per token: the gate formula's derivative plus
//   the load-balance and z-loss terms, written to dZ [n, E];
// * a grouped bf16 GEMM on v_mfma_f32_16x16x32_bf16 for every product of
//   the expert FFN and router backward.  Groups split either the rows (the
//   expert-major buffer: pre-activation recompute, dH, dX, router dX) or K
//   (weight gradients: a sum over an expert's rows).  Each operand is staged
//   into LDS per 32-wide K step as it is stored: a K-contiguous operand as
//   [row][K] and read with 16-byte loads, a K-strided one (K is its row
//   index: W2 and W1 in dH = dY W2 and dX = dA W1, and both operands of a
//   weight gradient) as [K][row] and read with ds_read_b64_tr_b16, whose
//   16-lane transpose hands each lane four consecutive K values of its own
//   column, so no copy is ever transposed in memory.  The activation
//   derivative is fused into the dH epilogue;
// * a plain fp32 grouped GEMM (one thread per output) for fp32 data and for
//   shapes the bf16 tiling does not cover.
#include <atomic>

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

typedef __bf16 bwbf16x8_t __attribute__((ext_vector_type(8)));
typedef float bwf32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t bwu32x4_t __attribute__((ext_vector_type(4)));
typedef short bwv4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bwv4i16 bw_lds_v4i16;

// ------------------------------------------------------------------ helpers

MOE_DEV float load_f(const float* p) { return *p; }
MOE_DEV float load_f(const bf16_t* p) { return bf16_to_f32(*p); }
MOE_DEV void store_f(float* p, float v) { *p = v; }
MOE_DEV void store_f(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// GELU x Phi(x) with Phi from erff, and its derivative Phi(x) + x phi(x).
MOE_DEV float gelu_exact(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
MOE_DEV float gelu_exact_grad(float x) {
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.39894228040143268f * expf(-0.5f * x * x);
}
MOE_DEV float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// ------------------------------------------------------------ combine backward

// One wave per slot s < n_kept: t = slot_token[s], g = slot_gate[s];
// dY[s] = g * dOut[t] (fp32 product, one rounding), d_gate[s] = sum over
// columns of dOut[t] * Y[s]: each lane accumulates its columns in order with
// fmaf, then a halving tree over the lanes.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dout, const T* __restrict__ Y,
                                                          const int32_t* __restrict__ slot_token,
                                                          const float* __restrict__ slot_gate,
                                                          const int32_t* __restrict__ n_kept, int64_t M_max,
                                                          int d, T* __restrict__ dY, float* __restrict__ d_gate) {
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = min((int64_t)*n_kept, M_max);
  if (s >= rows) return;
  const int t = slot_token[s];
  const float g = slot_gate[s];
  const T* o = dout + (size_t)t * d;
  const T* y = Y + (size_t)s * d;
  T* dy = dY + (size_t)s * d;
  float dot = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float ov = load_f(o + c);
    store_f(dy + c, g * ov);
    dot = fmaf(ov, load_f(y + c), dot);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dot = dot + __shfl_down(dot, off, 64);
  if (lane == 0) d_gate[s] = dot;
}

// bf16 rows of whole 16-byte chunks: 8 columns per lane and chunk.
__global__ __launch_bounds__(256) void combine_bwd_vec_kernel(const bf16_t* __restrict__ dout,
                                                              const bf16_t* __restrict__ Y,
                                                              const int32_t* __restrict__ slot_token,
                                                              const float* __restrict__ slot_gate,
                                                              const int32_t* __restrict__ n_kept, int64_t M_max,
                                                              int d, bf16_t* __restrict__ dY,
                                                              float* __restrict__ d_gate) {
  const int lane = threadIdx.x & 63;
  const int64_t s = __builtin_amdgcn_readfirstlane((int)((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int64_t rows = min((int64_t)*n_kept, M_max);
  if (s >= rows) return;
  const int t = slot_token[s];
  const float g = slot_gate[s];
  const bwu32x4_t* o = reinterpret_cast<const bwu32x4_t*>(dout + (size_t)t * d);
  const bwu32x4_t* y = reinterpret_cast<const bwu32x4_t*>(Y + (size_t)s * d);
  bwu32x4_t* dy = reinterpret_cast<bwu32x4_t*>(dY + (size_t)s * d);
  const int nv = d / 8;
  float dot = 0.f;
  for (int c = lane; c < nv; c += 64) {
    const bwu32x4_t ov = o[c], yv = y[c];
    bwu32x4_t out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o0 = __uint_as_float(ov[i] << 16), o1 = __uint_as_float(ov[i] & 0xFFFF0000u);
      const float y0 = __uint_as_float(yv[i] << 16), y1 = __uint_as_float(yv[i] & 0xFFFF0000u);
      out[i] = pack_bf16x2(g * o0, g * o1);
      dot = fmaf(o0, y0, dot);
      dot = fmaf(o1, y1, dot);
    }
    dy[c] = out;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dot = dot + __shfl_down(dot, off, 64);
  if (lane == 0) d_gate[s] = dot;
}

hipError_t launch_combine_backward(const void* dout, const void* Y, int dtype, int d, const int32_t* slot_token,
                                   const float* slot_gate, const int32_t* n_kept, int64_t M_max, void* dY,
                                   float* d_gate, hipStream_t stream) {
  if (M_max <= 0) return hipSuccess;
  const dim3 grid((unsigned)((M_max + 3) / 4)), block(256);
  if (dtype == 1 && d % 8 == 0)
    hipLaunchKernelGGL(combine_bwd_vec_kernel, grid, block, 0, stream, static_cast<const bf16_t*>(dout),
                       static_cast<const bf16_t*>(Y), slot_token, slot_gate, n_kept, M_max, d,
                       static_cast<bf16_t*>(dY), d_gate);
  else if (dtype == 1)
    hipLaunchKernelGGL(combine_bwd_kernel<bf16_t>, grid, block, 0, stream, static_cast<const bf16_t*>(dout),
                       static_cast<const bf16_t*>(Y), slot_token, slot_gate, n_kept, M_max, d,
                       static_cast<bf16_t*>(dY), d_gate);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, grid, block, 0, stream, static_cast<const float*>(dout),
                       static_cast<const float*>(Y), slot_token, slot_gate, n_kept, M_max, d,
                       static_cast<float*>(dY), d_gate);
  return hipGetLastError();
}

// --------------------------------------------------------------- gate backward

// One wave per token, lane l holds experts l + 64 j (j < NJ).  dz starts
// from the gate formula's derivative (selected experts only, through a
// per-wave LDS row so that lane q's contribution reaches the lane owning
// expert idx[q]; the k experts of a token are distinct), then adds
// p (c - <p, c>) for the load-balance loss (c_e = lb_coef E f_e / n;
// scores: through r / sum r) and z_coef (2 / n) lse p for the z-loss.
constexpr int kGateRows = 16;

template <int NJ>
__global__ __launch_bounds__(1024) void gate_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ sel_idx, const float* __restrict__ d_gate,
    const int32_t* __restrict__ assign_slot, const int32_t* __restrict__ token_offset,
    const int32_t* __restrict__ token_slot, const int32_t* __restrict__ expert_count, int n, int E, int k,
    int dir, int score, int norm_topk, float lb_coef, float z_coef, float* __restrict__ dZ) {
  __shared__ float s_c[kMaxExperts];
  __shared__ float s_row[kGateRows][64 * NJ];
  __shared__ float s_tot;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // load-balance weights c_e = lb_coef * E * f_e / n, f_e = count_e / sum(count)
  if (wave == 0) {
    float tot = 0.f;
    for (int e = lane; e < E; e += 64) tot += (float)expert_count[e];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o, 64);
    if (lane == 0) s_tot = tot;
  }
  for (int j = lane; j < 64 * NJ; j += 64) s_row[wave][j] = 0.f;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024)
    s_c[e] = s_tot > 0.f ? lb_coef * (float)E * ((float)expert_count[e] / s_tot) / (float)n : 0.f;
  __syncthreads();
  const int t = blockIdx.x * kGateRows + wave;
  if (t >= n) return;
  float z[NJ], p[NJ];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    z[j] = e < E ? logits[(size_t)t * E + e] : -__builtin_huge_valf();
    m = fmaxf(m, z[j]);
  }
  m = wave_max_f32(m);
  float ssum = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    p[j] = lane + 64 * j < E ? expf(z[j] - m) : 0.f;
    ssum += p[j];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ssum += __shfl_xor(ssum, o, 64);
#pragma unroll
  for (int j = 0; j < NJ; ++j) p[j] = p[j] / ssum;
  const float lse = m + logf(ssum);
  float* row = s_row[wave];

  if (dir == 0) {
    // lane q < k: the token's q-th choice
    const bool on = lane < k;
    const int e_q = on ? sel_idx[(size_t)t * k + lane] : 0;
    const int a_q = on ? assign_slot[(size_t)t * k + lane] : -1;
    const float dg = a_q >= 0 ? d_gate[a_q] : 0.f;
    const float zq = on ? logits[(size_t)t * E + e_q] : 0.f;
    if (score == 0 && !norm_topk) {
      // full-row softmax probability: dp at the chosen experts
      if (on) row[e_q] = dg;
    } else {
      float dzq;
      if (score == 0) {
        float mq = on ? zq : -__builtin_huge_valf();
        mq = wave_max_f32(mq);
        const float eq = on ? expf(zq - mq) : 0.f;
        float sq = eq;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
        const float gq = eq / sq;
        float sgd = gq * dg;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sgd += __shfl_xor(sgd, o, 64);
        dzq = gq * (dg - sgd);
      } else {
        const float sg = sigm(zq);
        const float r = score == 1 ? sg : sqrtf(fmaxf(zq, 0.f) + log1pf(expf(-fabsf(zq))));
        const float rp = score == 1 ? sg * (1.f - sg) : sg / (2.f * r);
        float dr = dg;
        if (norm_topk) {
          float R = on ? r : 0.f;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) R += __shfl_xor(R, o, 64);
          const float gq = r / R;
          float sgd = on ? gq * dg : 0.f;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) sgd += __shfl_xor(sgd, o, 64);
          dr = (dg - sgd) / R;
        }
        dzq = dr * rp;
      }
      if (on) row[e_q] = dzq;
    }
  } else {
    // expert choice: dS at the experts whose slots are in the token's list
    const int q0 = token_offset[t], q1 = token_offset[t + 1];
    for (int q = q0 + lane; q < q1; q += 64) {
      const int s = token_slot[q];
      if (s >= 0) row[s / k] = d_gate[s];
    }
  }
  // one wave's LDS writes are visible to its later reads
  float dz[NJ], g_in[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) g_in[j] = row[lane + 64 * j];
  const bool through_softmax = dir == 1 || (score == 0 && !norm_topk);
  float pd = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) pd += p[j] * g_in[j];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) pd += __shfl_xor(pd, o, 64);
#pragma unroll
  for (int j = 0; j < NJ; ++j) dz[j] = through_softmax ? p[j] * (g_in[j] - pd) : g_in[j];
  // load-balance loss
  if (lb_coef != 0.f && s_tot > 0.f) {
    float c[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) c[j] = lane + 64 * j < E ? s_c[lane + 64 * j] : 0.f;
    if (score == 0) {
      float pc = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) pc += p[j] * c[j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) pc += __shfl_xor(pc, o, 64);
#pragma unroll
      for (int j = 0; j < NJ; ++j) dz[j] += p[j] * (c[j] - pc);
    } else {
      float r[NJ], rp[NJ];
      float R = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool v = lane + 64 * j < E;
        const float sg = sigm(z[j]);
        r[j] = !v ? 0.f : score == 1 ? sg : sqrtf(fmaxf(z[j], 0.f) + log1pf(expf(-fabsf(z[j]))));
        rp[j] = !v ? 0.f : score == 1 ? sg * (1.f - sg) : sg / (2.f * r[j]);
        R += r[j];
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) R += __shfl_xor(R, o, 64);
      float pc = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) pc += (r[j] / R) * c[j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) pc += __shfl_xor(pc, o, 64);
#pragma unroll
      for (int j = 0; j < NJ; ++j) dz[j] += rp[j] * (c[j] - pc) / R;
    }
  }
  if (z_coef != 0.f) {
    const float zc = z_coef * (2.f / (float)n) * lse;
#pragma unroll
    for (int j = 0; j < NJ; ++j) dz[j] += zc * p[j];
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    if (e < E) dZ[(size_t)t * E + e] = dz[j];
  }
}

hipError_t launch_gate_backward(const float* logits, const int32_t* sel_idx, const float* d_gate,
                                const MapPtrs& m, int n, int E, int k, int dir, int score, int norm_topk,
                                float lb_coef, float z_coef, float* dZ, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((n + kGateRows - 1) / kGateRows), block(1024);
  const auto kern = E <= 64 ? gate_bwd_kernel<1> : E <= 128 ? gate_bwd_kernel<2>
                    : E <= 256 ? gate_bwd_kernel<4> : gate_bwd_kernel<8>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, logits, sel_idx, d_gate, m.assign_slot, m.token_offset,
                     m.token_slot, m.expert_count, n, E, k, dir, score, norm_topk, lb_coef, z_coef, dZ);
  return hipGetLastError();
}

// ------------------------------------------------------------- grouped GEMM

// C(i, j) = sum_k A(i, k) B(k, j).  A(i, k) = A[i * lda + k] when kAK (K
// contiguous) else A[k * lda + i]; B(k, j) = B[j * ldb + k] when kBK else
// B[k * ldb + j].
//   Row-grouped (kMode 0): group g owns rows offsets[g] .. offsets[g+1]-1 of
//   A and C (absolute row indices); B of group g starts at B + g *
//   b_stride; K = args.K; J columns.
//   K-grouped (kMode 1): group g sums over k = offsets[g] .. offsets[g+1]-1
//   (rows of A and B), C of group g starts at C + g * c_stride and has
//   I x J entries.
struct GemmArgs {
  const bf16_t* A;
  int64_t lda;
  const bf16_t* B;
  int64_t ldb;
  int64_t b_stride;
  void* C;
  int64_t ldc;
  int64_t c_stride;
  const int32_t* offsets;
  int groups, I, J, K;
  const bf16_t* base;  // EPI_BF16_ADD: C = base + A B (ld = ldc)
  const float* pre;    // activation backward: fp32 pre-activations [rows, ld_pre]
  int64_t ld_pre;
  bf16_t* h_out;       // activation backward: act(pre) [rows, ld_h]
  int64_t ld_h;
  int f;               // activation backward: hidden size (SwiGLU up columns start at f)
  // weight gradients: per-XCD expert lists from wgrad_plan_kernel, or
  // nullptr for equal tile counts per XCD
  const int32_t* plan;
};

enum { EPI_BF16 = 0, EPI_BF16_ADD = 1, EPI_F32 = 2, EPI_GELU_BWD = 3, EPI_SWIGLU_BWD = 4 };

// Which GEMM outputs are written with non-temporal stores (bit 0: the fp32
// pre-activation, bit 1: the fp32 weight gradients, bit 2: bf16 outputs),
// and whether a weight-gradient tile goes out through LDS in whole rows.
#ifndef MOE_BW_NT
#define MOE_BW_NT 3
#endif
#ifndef MOE_BW_STAGE_DW
#define MOE_BW_STAGE_DW 1
#endif
// Row-grouped GEMMs on 128 x 256 tiles when the experts average at least
// MOE_BW_WIDE_ROWS rows (the host's row bound over the groups)
#ifndef MOE_BW_WIDE
#define MOE_BW_WIDE 1
#endif
#ifndef MOE_BW_WIDE_ROWS
#define MOE_BW_WIDE_ROWS 512
#endif
// Weight gradients with whole-tile J on the persistent kernel
#ifndef MOE_BW_PERSIST
#define MOE_BW_PERSIST 1
#endif

template <bool kNT, typename V>
MOE_DEV void vstore(V* p, V v) {
  if (kNT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Epilogue of one output element (row `r`, column `c`, value v); row-grouped
// rows are absolute, K-grouped outputs start at the group's C.
template <int kEpi>
MOE_DEV void epi_store(const GemmArgs& a, void* Cg, int64_t r, int c, float v) {
#pragma clang fp contract(off)
  if (kEpi == EPI_F32) {
    static_cast<float*>(Cg)[r * a.ldc + c] = v;
  } else if (kEpi == EPI_BF16) {
    static_cast<bf16_t*>(Cg)[r * a.ldc + c] = f32_to_bf16(v);
  } else if (kEpi == EPI_BF16_ADD) {
    const float b = a.base ? bf16_to_f32(a.base[r * a.ldc + c]) : 0.f;
    static_cast<bf16_t*>(Cg)[r * a.ldc + c] = f32_to_bf16(b + v);
  } else if (kEpi == EPI_GELU_BWD) {
    const float x = a.pre[r * a.ld_pre + c];
    static_cast<bf16_t*>(Cg)[r * a.ldc + c] = f32_to_bf16(v * gelu_exact_grad(x));
    a.h_out[r * a.ld_h + c] = f32_to_bf16(gelu_exact(x));
  } else {
    const float gp = a.pre[r * a.ld_pre + c];
    const float up = a.pre[r * a.ld_pre + a.f + c];
    const float sg = sigm(gp);
    const float si = gp * sg;
    static_cast<bf16_t*>(Cg)[r * a.ldc + c] = f32_to_bf16(v * up * (sg * (1.f + gp * (1.f - sg))));
    static_cast<bf16_t*>(Cg)[r * a.ldc + a.f + c] = f32_to_bf16(v * si);
    a.h_out[r * a.ld_h + c] = f32_to_bf16(si * up);
  }
}

// Four consecutive columns c .. c+3 of row r (the row pitches are multiples
// of 4 elements, so the accesses are 16-byte (fp32) or 8-byte (bf16)
// aligned).
typedef uint32_t bwu32x2_t __attribute__((ext_vector_type(2)));
template <int kEpi, bool kNT>
MOE_DEV void epi_store4(const GemmArgs& a, void* Cg, int64_t r, int c, bwf32x4_t v) {
#pragma clang fp contract(off)
  if (kEpi == EPI_F32) {
    vstore<kNT>(reinterpret_cast<bwf32x4_t*>(static_cast<float*>(Cg) + r * a.ldc + c), v);
  } else if (kEpi == EPI_BF16) {
    vstore<kNT>(reinterpret_cast<bwu32x2_t*>(static_cast<bf16_t*>(Cg) + r * a.ldc + c),
                bwu32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
  } else if (kEpi == EPI_BF16_ADD) {
    if (a.base) {
      const bwu32x2_t b = *reinterpret_cast<const bwu32x2_t*>(a.base + r * a.ldc + c);
      v[0] = __uint_as_float(b[0] << 16) + v[0];
      v[1] = __uint_as_float(b[0] & 0xFFFF0000u) + v[1];
      v[2] = __uint_as_float(b[1] << 16) + v[2];
      v[3] = __uint_as_float(b[1] & 0xFFFF0000u) + v[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = 0.f + v[e];
    }
    vstore<kNT>(reinterpret_cast<bwu32x2_t*>(static_cast<bf16_t*>(Cg) + r * a.ldc + c),
                bwu32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
  } else if (kEpi == EPI_GELU_BWD) {
    const bwf32x4_t x = *reinterpret_cast<const bwf32x4_t*>(a.pre + r * a.ld_pre + c);
    float da[4], h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      da[e] = v[e] * gelu_exact_grad(x[e]);
      h[e] = gelu_exact(x[e]);
    }
    vstore<kNT>(reinterpret_cast<bwu32x2_t*>(static_cast<bf16_t*>(Cg) + r * a.ldc + c),
                bwu32x2_t{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])});
    vstore<kNT>(reinterpret_cast<bwu32x2_t*>(a.h_out + r * a.ld_h + c),
                bwu32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])});
  } else {
    const bwf32x4_t gp = *reinterpret_cast<const bwf32x4_t*>(a.pre + r * a.ld_pre + c);
    const bwf32x4_t up = *reinterpret_cast<const bwf32x4_t*>(a.pre + r * a.ld_pre + a.f + c);
    float dg[4], du[4], h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sg = sigm(gp[e]);
      const float si = gp[e] * sg;
      dg[e] = v[e] * up[e] * (sg * (1.f + gp[e] * (1.f - sg)));
      du[e] = v[e] * si;
      h[e] = si * up[e];
    }
    bf16_t* C = static_cast<bf16_t*>(Cg) + r * a.ldc;
    vstore<kNT>(reinterpret_cast<bwu32x2_t*>(C + c), bwu32x2_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])});
    vstore<kNT>(reinterpret_cast<bwu32x2_t*>(C + a.f + c),
                bwu32x2_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])});
    vstore<kNT>(reinterpret_cast<bwu32x2_t*>(a.h_out + r * a.ld_h + c),
                bwu32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])});
  }
}

// Workgroups are dealt to the 8 XCDs round-robin by linear id, and each XCD
// has its own L2.  Tile t of n goes to workgroup b so that XCD b % 8 owns a
// contiguous range of tiles (the first n % 8 XCDs one more): tiles that
// share an operand band (the column tiles of one row tile) then share one
// L2 instead of fetching the band once per XCD.
#ifndef MOE_BW_XCD
#define MOE_BW_XCD 1
#endif
constexpr int kBwXcds = 8;
MOE_DEV int xcd_range_start(int n, int xcd) {
  const int q = n / kBwXcds, r = n % kBwXcds;
  return xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
}
MOE_DEV int xcd_tile(int n, int b) {
  return MOE_BW_XCD ? xcd_range_start(n, b % kBwXcds) + b / kBwXcds : b;
}

// Schedule of the persistent weight-gradient kernels.  A tile's time grows
// with its expert's row count (the K of its product), and routed loads are
// skewed (the top-8 Zipf workload's largest expert has 8x the mean), so an
// equal count of tiles per XCD and per workgroup leaves most of the chip
// idle while a few workgroups finish the largest experts.  This kernel (one
// workgroup, before the weight gradients) deals whole experts to the 8 XCDs,
// longest first, each to the XCD with the least work so far, so that an
// expert's operand bands stay in one L2.  In the kernels the k workgroups of
// an XCD take the tiles of its list round-robin (positions w, w + k, ...),
// longest experts first: within a few percent of an even split, with no
// atomics (whose returns would have to wait behind the loads in flight).
// Cost of a tile: its 32-row K steps (rounds of two, at least one) plus 16
// for the output.  plan[x * groups + k]: k-th expert of XCD x;
// plan[8 groups + x]: their count.
constexpr int kPlanThreads = kMaxExperts;
__global__ __launch_bounds__(kPlanThreads) void wgrad_plan_kernel(const int32_t* __restrict__ offsets, int groups,
                                                                  int32_t* __restrict__ plan) {
  __shared__ int cost[kPlanThreads], order[kPlanThreads];
  const int e = threadIdx.x;
  int c = 0;
  if (e < groups) {
    const int k = offsets[e + 1] - offsets[e];
    c = 2 * max(1, (k + 63) / 64) + 16;
  }
  cost[e] = c;
  __syncthreads();
  if (e < groups) {
    int rank = 0;                                  // longest first, lower index first among equals
    for (int o = 0; o < groups; ++o) {
      const int co = cost[o];
      rank += (co > c || (co == c && o < e)) ? 1 : 0;
    }
    order[rank] = e;
  }
  __syncthreads();
  if (e < 64) {
    // wave 0 deals the experts in rank order.  Lane l holds ranks l, l + 64,
    // ...; lanes 0..7 hold the running work and list length of XCDs 0..7.
    // Per expert: the least-loaded XCD (lowest index among equals) by a
    // minimum of load * 8 + x over lanes 0..7 (three row shifts: lane 7 ends
    // with the minimum), then that lane adds the expert's cost.  Loads stay
    // below 2^28 (the costs sum to at most M_max / 32 + 16 E).
    constexpr int kChunks = kPlanThreads / 64;
    int og[kChunks], oc[kChunks], myx[kChunks], myp[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int r = c * 64 + e;
      og[c] = r < groups ? order[r] : 0;
      oc[c] = r < groups ? cost[og[c]] : 0;
      myx[c] = 0;
      myp[c] = 0;
    }
    int ld = 0, cn = 0;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int lim = min(64, groups - c * 64);
      for (int l = 0; l < lim; ++l) {
        const int cg = __builtin_amdgcn_readlane(oc[c], l);
        int key = e < kBwXcds ? ld * kBwXcds + e : INT32_MAX;
        key = min(key, __builtin_amdgcn_update_dpp(INT32_MAX, key, 0x111, 0xf, 0xf, false));   // row_shr:1
        key = min(key, __builtin_amdgcn_update_dpp(INT32_MAX, key, 0x112, 0xf, 0xf, false));   // row_shr:2
        key = min(key, __builtin_amdgcn_update_dpp(INT32_MAX, key, 0x114, 0xf, 0xf, false));   // row_shr:4
        const int best = __builtin_amdgcn_readlane(key, kBwXcds - 1) & (kBwXcds - 1);
        const int pos = __builtin_amdgcn_readlane(cn, best);
        if (e == best) ld += cg, cn += 1;
        if (e == l) myx[c] = best, myp[c] = pos;
      }
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      if (c * 64 + e < groups) plan[myx[c] * groups + myp[c]] = og[c];
    if (e < kBwXcds) plan[8 * groups + e] = cn;
  }
}

// A weight-gradient workgroup's tile sequence.  With a plan: position p of
// its XCD's list (copied to LDS once, so that no wait in the tile loop is a
// memory wait) is tile (list[p / per_group], p % per_group), in the global
// numbering (g tiles_i + ti) tiles_j + tj; positions w, w + k, ... for the
// w-th of the XCD's k workgroups.  Without: the equal split by tile count.
struct WgradSchedule {
  int* list;                                       // LDS, kMaxExperts entries
  int n, per_group, step, t_end;
  bool dyn;
  MOE_DEV int first(const GemmArgs& a, int total) {
    const int xcd = blockIdx.x % kBwXcds;
    const bool by_xcd = MOE_BW_XCD && gridDim.x % kBwXcds == 0;
    dyn = a.plan != nullptr && by_xcd;
    if (dyn) {
      const int cnt = a.plan[8 * a.groups + xcd];
      for (int i = threadIdx.x; i < cnt; i += blockDim.x) list[i] = a.plan[xcd * a.groups + i];
      __syncthreads();
      n = cnt * per_group;
      step = gridDim.x / kBwXcds;
      return at((int)blockIdx.x / kBwXcds);
    }
    step = by_xcd ? gridDim.x / kBwXcds : gridDim.x;
    t_end = by_xcd ? xcd_range_start(total, xcd + 1) : total;
    const int t = by_xcd ? xcd_range_start(total, xcd) + blockIdx.x / kBwXcds : blockIdx.x;
    return t < t_end ? t : -1;
  }
  // tile at position p (dyn) or -1 past the end
  MOE_DEV int at(int p) const { return p < n ? list[p / per_group] * per_group + p % per_group : -1; }
};

// Locate the row-grouped tile of linear workgroup id b over nJ column
// tiles: group g, its 128-row tile index and the column tile, or g = -1
// past the live tiles.  Lane l of wave 0 counts the row tiles of a
// contiguous run of groups; a wave scan gives every run its first tile and
// the total, over which the tiles are spread across the XCDs (b < nJ x
// total; the grid's slots beyond return at once).
MOE_DEV void locate_row_tile(const int32_t* __restrict__ offsets, int G, int nJ, int b, int* s_g, int* s_tile,
                             int* s_x) {
  const int lane = threadIdx.x & 63;
  const int per = (G + 63) / 64;
  const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
  int cnt = 0;
  for (int g = g0; g < g1; ++g) cnt += (offsets[g + 1] - offsets[g] + 127) >> 7;
  const int incl = wave_inclusive_scan_i32(cnt);
  const int n = nJ * __builtin_amdgcn_readlane(incl, 63);
  int base = incl - cnt;
  if (lane == 0) *s_g = -1;
  __builtin_amdgcn_wave_barrier();
  if (b >= n) return;
  const int t = xcd_tile(n, b);
  const int bx = t / nJ;
  if (bx >= base && bx < incl) {
    for (int g = g0; g < g1; ++g) {
      const int tiles = (offsets[g + 1] - offsets[g] + 127) >> 7;
      if (bx < base + tiles) {
        *s_g = g;
        *s_tile = bx - base;
        *s_x = t % nJ;
        break;
      }
      base += tiles;
    }
  }
}

// LDS stages, laid out so that no access conflicts on the 64 banks:
// * K-contiguous [128][32] (64-byte rows, no padding), the 16-byte chunk c
//   of row r stored at chunk c ^ ((r / 4) % 4): a store pass (4 rows x 64
//   bytes) and a fragment read (16 rows, one chunk each) both cover every
//   bank once;
// * K-strided [32][136] (272-byte rows, 4 banks apart), K row k stored at
//   row 8 (k / 8) + 2 (k % 4) + (k % 8) / 4: the 4 K rows a 16-lane group
//   of a transpose read touches (k0 .. k0+3, or k0+4 .. k0+7) start 8 banks
//   apart, and the two groups of a 32-lane pass 32 banks apart.
constexpr int kGT = 128;             // tile rows and columns
constexpr int kGK = 32;              // K per step
constexpr int kLdKc = kGK;           // LDS stride (bf16) of a K-contiguous stage [128][32]
constexpr int kLdKs = kGT + 8;       // LDS stride of a K-strided stage [32][136]
constexpr int kStageElems = 32 * kLdKs;   // 4352 >= 128 * 32

MOE_DEV int kc_lds(int r, int chunk) { return r * kLdKc + ((chunk ^ ((r >> 2) & 3)) << 3); }
MOE_DEV int ks_row(int k) { return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1); }
#ifndef MOE_BW_RING
#define MOE_BW_RING 4
#endif
constexpr int kBwRing = MOE_BW_RING;        // K steps of operands in registers (even)

// One 128 x 128 output tile's K loop: acc = sum over k < klen of
// A[i0 + i, k] B[j0 + j, k] (C^T fragments).  abase / bbase and their byte
// bounds locate the operands (reads past the bounds return zero);
// kAK / kBK say whether an operand is K-contiguous ([row][K], leading
// dimension lda / ldb) or K-strided ([K][row]).  All 256 threads call it.
template <bool kAK, bool kBK, int R = kBwRing>
MOE_DEV void tile_mainloop(const bf16_t* abase, int64_t abytes, int64_t lda, int i0, const bf16_t* bbase,
                           int64_t bbytes, int64_t ldb, int j0, int klen, bf16_t (*sA)[kStageElems],
                           bf16_t (*sB)[kStageElems], bwf32x4_t (&acc)[4][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int ns = (klen + kGK - 1) / kGK;
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(abase), (short)0, (int)min(abytes, (int64_t)0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(bbase), (short)0, (int)min(bbytes, (int64_t)0x7FFFFFFF), 0x00020000);

  // Per step each thread moves two 16-byte chunks of each operand.
  //   K-contiguous: chunk c -> row c / 4 of the tile, K offset 8 (c % 4);
  //   K-strided:    chunk c -> K row c / 16, column offset 8 (c % 16).
  int a_off[2], b_off[2], a_lds[2], b_lds[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 256 * h;
    if (kAK) {
      const int r = c >> 2, kq = (c & 3) * 8;
      a_off[h] = (int)(((int64_t)(i0 + r) * lda + kq) * 2);
      a_lds[h] = kc_lds(r, c & 3);
    } else {
      const int kr = c >> 4, ic = (c & 15) * 8;
      a_off[h] = (int)(((int64_t)kr * lda + i0 + ic) * 2);
      a_lds[h] = ks_row(kr) * kLdKs + ic;
    }
    if (kBK) {
      const int r = c >> 2, kq = (c & 3) * 8;
      b_off[h] = (int)(((int64_t)(j0 + r) * ldb + kq) * 2);
      b_lds[h] = kc_lds(r, c & 3);
    } else {
      const int kr = c >> 4, jc = (c & 15) * 8;
      b_off[h] = (int)(((int64_t)kr * ldb + j0 + jc) * 2);
      b_lds[h] = ks_row(kr) * kLdKs + jc;
    }
  }
  // scalar step offsets (bytes): K-contiguous operands advance along the
  // row, K-strided ones by 32 rows
  const int a_step = kAK ? kGK * 2 : (int)(kGK * lda * 2);
  const int b_step = kBK ? kGK * 2 : (int)(kGK * ldb * 2);
  // A ring of kBwRing steps in registers: the loads of the next kBwRing - 1
  // steps are in flight while one is multiplied.  The step count is padded
  // to a multiple of the ring; padded steps read zeros (K-contiguous tails
  // are zeroed below, K-strided rows past K lie outside the resource), so
  // every round runs whole and the loop has no branch.
  const int ns_pad = (ns + R - 1) / R * R;
  bwu32x4_t ra[R][2], rb[R][2];
  auto load = [&](int st, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[q][h] = __builtin_amdgcn_raw_buffer_load_b128(ar, a_off[h], st * a_step, 0);
      rb[q][h] = __builtin_amdgcn_raw_buffer_load_b128(br, b_off[h], st * b_step, 0);
    }
    // K-contiguous operands: K columns past K must be zero
    if (kAK || kBK) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kq = ((tid + 256 * h) & 3) * 8;
        const bool in = st * kGK + kq < klen;
        if (kAK && !in) ra[q][h] = bwu32x4_t{0u, 0u, 0u, 0u};
        if (kBK && !in) rb[q][h] = bwu32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store = [&](int q, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<bwu32x4_t*>(&sA[buf][a_lds[h]]) = ra[q][h];
      *reinterpret_cast<bwu32x4_t*>(&sB[buf][b_lds[h]]) = rb[q][h];
    }
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = bwf32x4_t{0.f, 0.f, 0.f, 0.f};
  // fragment offsets: K-contiguous stage -> row (lane % 16), K chunk
  // lane / 16 (row bases are multiples of 16, so the swizzle depends on the
  // lane only); K-strided stage -> transpose reads of K rows 8 (lane / 16) +
  // (lane % 16) / 4 (then + 4), column 4 (lane % 4), at their permuted rows
  const int kc_off = kc_lds(lane & 15, lane >> 4);
  const int ks_off = (8 * (lane >> 4) + 2 * ((lane >> 2) & 3)) * kLdKs + 4 * (lane & 3);
  auto frag = [&](const bf16_t* s, bool kcontig, int rowbase) -> bwbf16x8_t {
    if (kcontig) return *reinterpret_cast<const bwbf16x8_t*>(s + kc_off + rowbase * kLdKc);
    const bwv4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_off + rowbase));
    const bwv4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_off + kLdKs + rowbase));
    return __builtin_bit_cast(bwbf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // one K step from ring entry q; `next` >= 0 refills the entry with that
  // step's loads (the last round refills nothing)
  auto step = [&](int q, int next) {
    // LDS buffer q % 2 was last read by step q - 2, which every wave
    // finished before the previous step's barrier
    const int buf = q & 1;
    store(q, buf);
    __syncthreads();
    if (next >= 0) load(next, q);
    bwbf16x8_t fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag(sA[buf], kAK, 64 * wr + 16 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = frag(sB[buf], kBK, 64 * wc + 16 * j);
    // B fragments as the first operand: the result is the C^T tile, so
    // each lane ends with 4 consecutive columns of one row of C
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int q = 0; q < R; ++q) load(q, q);
  for (int st0 = 0; st0 < ns_pad - R; st0 += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) step(q, st0 + q + R);
  }
#pragma unroll
  for (int q = 0; q < R; ++q) step(q, -1);
}

template <bool kAK, bool kBK, int kMode, int kEpi>
__global__ __launch_bounds__(256) void bw_gemm_bf16_kernel(GemmArgs a) {
  // operand stages; a weight-gradient epilogue reuses them for half a tile
  // of fp32 output
  __shared__ __attribute__((aligned(16))) bf16_t sAB[4][kStageElems];
  bf16_t(*sA)[kStageElems] = sAB;
  bf16_t(*sB)[kStageElems] = sAB + 2;
  __shared__ int s_g, s_tile, s_x;
  constexpr bool kNT = kEpi == EPI_F32 ? ((MOE_BW_NT >> (kMode == 1 ? 1 : 0)) & 1) != 0 : (MOE_BW_NT & 4) != 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;   // 2 x 2 waves of 64 x 64

  // column tiles fastest, so concurrent workgroups touch adjacent column
  // bands of the same rows (weights and outputs alike) instead of one band
  // of many rows a full row pitch apart
  int g, i0, j0 = blockIdx.x * kGT;
  int64_t row0 = 0;       // row-grouped: first absolute row of the tile
  int rows = kGT;         // row-grouped: valid rows of the tile
  int kbeg = 0, klen = a.K;
  if (kMode == 0) {
    if (wave == 0)
      locate_row_tile(a.offsets, a.groups, gridDim.x, blockIdx.x + blockIdx.y * gridDim.x, &s_g, &s_tile, &s_x);
    __syncthreads();
    g = s_g;
    if (g < 0) return;
    j0 = s_x * kGT;
    row0 = (int64_t)a.offsets[g] + (int64_t)s_tile * kGT;
    rows = min((int64_t)kGT, (int64_t)a.offsets[g + 1] - row0);
    i0 = 0;
  } else {
    g = blockIdx.z;
    i0 = blockIdx.y * kGT;
    kbeg = a.offsets[g];
    klen = a.offsets[g + 1] - kbeg;
  }
  void* Cg = kMode == 0 ? a.C
                        : (void*)((char*)a.C + (size_t)g * a.c_stride * (kEpi == EPI_F32 ? 4 : 2));
  const int ns = (klen + kGK - 1) / kGK;
  if (kMode == 1 && ns == 0) {
    // an expert without rows: zero gradient
    for (int e = tid; e < kGT * kGT; e += 256) {
      const int r = i0 + e / kGT, c = j0 + e % kGT;
      if (r < a.I && c < a.J) epi_store<kEpi>(a, Cg, r, c, 0.f);
    }
    return;
  }
  // buffer resources (bounds: rows past the group read as zero)
  const bf16_t* abase;
  int64_t abytes;
  if (kMode == 0) {
    abase = a.A + row0 * a.lda;
    abytes = (int64_t)rows * a.lda * 2;
  } else {
    abase = a.A + (int64_t)kbeg * a.lda;
    abytes = (int64_t)klen * a.lda * 2;
  }
  const bf16_t* bbase;
  int64_t bbytes;
  if (kMode == 0) {
    bbase = a.B + (int64_t)g * a.b_stride;
    bbytes = kBK ? (int64_t)a.J * a.ldb * 2 : (int64_t)a.K * a.ldb * 2;
  } else {
    bbase = a.B + (int64_t)kbeg * a.ldb;
    bbytes = (int64_t)klen * a.ldb * 2;
  }
  bwf32x4_t acc[4][4];
  tile_mainloop<kAK, kBK>(abase, abytes, a.lda, i0, bbase, bbytes, a.ldb, j0, klen, sA, sB, acc);
  // C^T fragment: lane holds row (lane % 16) of its 16 x 16 subtile and
  // columns 4 (lane / 16) .. +3; whole groups of 4 in-range columns go out
  // as one vector access (when the row pitches allow it), the rest element
  // by element
  if constexpr (kMode == 1 && kEpi == EPI_F32 && MOE_BW_STAGE_DW) {
    // Weight gradient: the tile goes out in two halves of 64 rows through
    // LDS (row stride 132 floats: the fragment writes of 16 rows land 4
    // banks apart), read back so that 32 consecutive lanes store one
    // 512-byte row, whole cache lines per store instead of 64-byte pieces
    // of 16 rows.
    float* sC = reinterpret_cast<float*>(&sAB[0][0]);
    constexpr int kCs = kGT + 4;
    static_assert(64 * kCs * 4 <= 4 * kStageElems * 2, "half tile fits the stages");
    const bool vec_out = a.ldc % 4 == 0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      __syncthreads();   // p = 0: the last step's fragment reads; p = 1: half 0's read-out
      if (wr == p) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<bwf32x4_t*>(sC + (16 * i + (lane & 15)) * kCs + 64 * wc + 16 * j + 4 * (lane >> 4)) =
                acc[i][j];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = tid + 256 * q;   // 64 rows x 32 chunks of 4
        const int r = e >> 5, c = (e & 31) * 4;
        const int gr = i0 + 64 * p + r, gc = j0 + c;
        if (gr >= a.I) continue;
        const bwf32x4_t v = *reinterpret_cast<const bwf32x4_t*>(sC + r * kCs + c);
        float* dst = static_cast<float*>(Cg) + (int64_t)gr * a.ldc + gc;
        if (vec_out && gc + 3 < a.J) {
          vstore<kNT>(reinterpret_cast<bwf32x4_t*>(dst), v);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (gc + u < a.J) dst[u] = v[u];
        }
      }
    }
    return;
  }
  const bool vec = a.ldc % 4 == 0 && (kEpi < EPI_GELU_BWD || (a.ld_pre % 4 == 0 && a.ld_h % 4 == 0));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ti = 64 * wr + 16 * i + (lane & 15);
      const int c = j0 + 64 * wc + 16 * j + 4 * (lane >> 4);
      const bool row_ok = kMode == 0 ? ti < rows : i0 + ti < a.I;
      const int64_t r = kMode == 0 ? row0 + ti : (int64_t)(i0 + ti);
      if (!row_ok) continue;
      if (vec && c + 3 < a.J) {
        epi_store4<kEpi, kNT>(a, Cg, r, c, acc[i][j]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < a.J) epi_store<kEpi>(a, Cg, r, c + e, acc[i][j][e]);
      }
    }
}

// GELU: dH = dY W2 fused with the pre-activation recompute A = X W1^T.
// Both contract over d into the same [rows, f] tile, so one workgroup runs
// the two K loops into two register tiles and its epilogue forms
// dA = dH gelu'(A) and H = gelu(A): the fp32 pre-activation never leaves
// registers.  Row-grouped (tiles located from expert_offset as in the tiled
// kernel); the arithmetic is that of the recompute GEMM followed by the dH
// GEMM, bit for bit.  a: A = dY (lda = d), B = W2 (ldb = f, b_stride d f),
// C = dA (ldc = f), h_out = H (ld_h = f), J = f, K = d.
#ifndef MOE_BW_FUSE_DH
#define MOE_BW_FUSE_DH 1
#endif
// register ring of the second K loop (the first tile is live beside it)
#ifndef MOE_BW_FUSE_RING
#define MOE_BW_FUSE_RING 2
#endif
// dA and H staged through LDS and stored as whole 16-byte row pieces
#ifndef MOE_BW_FUSE_STAGE
#define MOE_BW_FUSE_STAGE 1
#endif
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bw_dh_gelu_fused_kernel(
    GemmArgs a, const bf16_t* __restrict__ X,
                                                               const bf16_t* __restrict__ W1) {
  __shared__ __attribute__((aligned(16))) bf16_t sAB[4][kStageElems];
  bf16_t(*sA)[kStageElems] = sAB;
  bf16_t(*sB)[kStageElems] = sAB + 2;
  __shared__ int s_g, s_tile, s_x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  if (wave == 0)
    locate_row_tile(a.offsets, a.groups, gridDim.x, blockIdx.x + blockIdx.y * gridDim.x, &s_g, &s_tile, &s_x);
  __syncthreads();
  const int g = s_g;
  if (g < 0) return;
  const int j0 = s_x * kGT;
  const int64_t row0 = (int64_t)a.offsets[g] + (int64_t)s_tile * kGT;
  const int rows = (int)min((int64_t)kGT, (int64_t)a.offsets[g + 1] - row0);
  const int d = a.K, f = a.J;
  bwf32x4_t pre[4][4], acc[4][4];
  // A = X W1^T: X rows and W1[g] rows ([f][d]) are both K-contiguous
  tile_mainloop<true, true>(X + row0 * d, (int64_t)rows * d * 2, d, 0, W1 + (int64_t)g * f * d,
                            (int64_t)f * d * 2, d, j0, d, sA, sB, pre);
  __syncthreads();
  // dH = dY W2: W2[g] is [d][f], K-strided
  tile_mainloop<true, false, MOE_BW_FUSE_RING>(a.A + row0 * a.lda, (int64_t)rows * a.lda * 2, a.lda, 0,
                                               a.B + (int64_t)g * a.b_stride,
                             (int64_t)d * a.ldb * 2, a.ldb, j0, d, sA, sB, acc);
  bf16_t* dA = static_cast<bf16_t*>(a.C);
  if (MOE_BW_FUSE_STAGE) {
    // dA goes to LDS as it is computed, H waits in registers as bf16 pairs;
    // each tile then leaves through LDS (row stride 136: the fragment
    // writes of 16 rows land 4 banks apart) as 16-byte pieces of whole rows
    // (f is a multiple of 8 here)
    constexpr int kHs = kGT + 8;
    static_assert(kGT * kHs <= 4 * kStageElems, "a bf16 output tile fits the stages");
    bf16_t* sC = &sAB[0][0];
    uint32_t ph[4][4][2];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float da[4], h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          da[e] = acc[i][j][e] * gelu_exact_grad(pre[i][j][e]);
          h[e] = gelu_exact(pre[i][j][e]);
        }
        ph[i][j][0] = pack_bf16x2(h[0], h[1]);
        ph[i][j][1] = pack_bf16x2(h[2], h[3]);
        *reinterpret_cast<bwu32x2_t*>(sC + (64 * wr + 16 * i + (lane & 15)) * kHs + 64 * wc + 16 * j +
                                      4 * (lane >> 4)) = bwu32x2_t{pack_bf16x2(da[0], da[1]),
                                                                   pack_bf16x2(da[2], da[3])};
      }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p == 1) {
        __syncthreads();   // dA has been read out
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<bwu32x2_t*>(sC + (64 * wr + 16 * i + (lane & 15)) * kHs + 64 * wc + 16 * j +
                                          4 * (lane >> 4)) = bwu32x2_t{ph[i][j][0], ph[i][j][1]};
      }
      __syncthreads();
      bf16_t* dst = p == 0 ? dA : a.h_out;
      const int64_t ld = p == 0 ? a.ldc : a.ld_h;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = tid + 256 * q;   // 128 rows x 16 chunks of 8
        const int r = e >> 4, c = (e & 15) * 8;
        if (r < rows && j0 + c < f)
          *reinterpret_cast<bwu32x4_t*>(dst + (row0 + r) * ld + j0 + c) =
              *reinterpret_cast<const bwu32x4_t*>(sC + r * kHs + c);
      }
    }
    return;
  }
  const bool vec = a.ldc % 4 == 0 && a.ld_h % 4 == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ti = 64 * wr + 16 * i + (lane & 15);
      const int c = j0 + 64 * wc + 16 * j + 4 * (lane >> 4);
      if (ti >= rows) continue;
      const int64_t r = row0 + ti;
      float da[4], h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        da[e] = acc[i][j][e] * gelu_exact_grad(pre[i][j][e]);
        h[e] = gelu_exact(pre[i][j][e]);
      }
      if (vec && c + 3 < f) {
        *reinterpret_cast<bwu32x2_t*>(dA + r * a.ldc + c) = bwu32x2_t{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
        *reinterpret_cast<bwu32x2_t*>(a.h_out + r * a.ld_h + c) =
            bwu32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < f) {
            dA[r * a.ldc + c + e] = f32_to_bf16(da[e]);
            a.h_out[r * a.ld_h + c + e] = f32_to_bf16(h[e]);
          }
      }
    }
}

// Persistent weight-gradient GEMM (K grouped by expert, both operands
// K-strided, fp32 out): C_g[i, j] = sum over the rows k of group g of
// A[k, i] B[k, j].  Tiles are numbered column tile fastest, then row tile,
// then group; each XCD owns a contiguous range of them, walked by its
// workgroups in strides (so an operand band is fetched into one L2).  The K loop of one
// expert is short (its rows / 32 steps), so a tile is mostly load latency
// and 64 KB of stores; here the last round of each tile refills the
// register ring with the next tile's first steps, whose loads are in flight
// while this tile's output is staged through LDS and stored.  The stores are
// buffer stores bounded by the group's I x J output (whole tiles in J; rows
// past I are dropped by the bound), so every thread issues the same count
// and no wait for a refill load has to wait for them too.  Needs J a
// multiple of 128 and ldc == J.
#ifndef MOE_WG_RING
#define MOE_WG_RING 4
#endif
#ifndef MOE_WG_WAVES
#define MOE_WG_WAVES 3
#endif
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MOE_WG_WAVES))) void bw_wgrad_bf16_kernel(
    GemmArgs a, int tiles_i, int tiles_j, int total) {
  __shared__ __attribute__((aligned(16))) bf16_t sAB[4][kStageElems];
  bf16_t(*sA)[kStageElems] = sAB;
  bf16_t(*sB)[kStageElems] = sAB + 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  constexpr int R = MOE_WG_RING;
  constexpr int kCs = 68;   // fp32 LDS row stride of the staged output
  static_assert(128 * kCs * 4 <= 4 * kStageElems * 2, "staged output fits the stages");
  // this workgroup's tiles: with a grid of whole XCD rounds, a strided walk
  // over its XCD's contiguous range, else over all tiles
  __shared__ int s_list[kMaxExperts];
  WgradSchedule sched;
  sched.list = s_list;
  sched.per_group = tiles_i * tiles_j;
  int t = sched.first(a, total);                   // uniform
  int pos = blockIdx.x / kBwXcds;                  // list position of tile t (plan)
  if (t < 0) return;

  // per thread and step: two 16-byte chunks of each operand, chunk c ->
  // K row c / 16, column offset 8 (c % 16); the tile's first column goes
  // into the scalar offset
  int a_off[2], b_off[2], s_lds[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 256 * h;
    const int kr = c >> 4, cc = (c & 15) * 8;
    a_off[h] = (int)(((int64_t)kr * a.lda + cc) * 2);
    b_off[h] = (int)(((int64_t)kr * a.ldb + cc) * 2);
    s_lds[h] = ks_row(kr) * kLdKs + cc;
  }
  const int a_step = (int)(kGK * a.lda * 2), b_step = (int)(kGK * a.ldb * 2);

  struct Tile {
    __amdgpu_buffer_rsrc_t ar, br;
    int g, i0, j0, klen;
  };
  // tile coordinates and operand resources (rows past the group's K read
  // as zero; `live` false gives empty resources, whose loads return zeros)
  auto tile_at = [&](int tt, bool live) -> Tile {
    Tile x;
    x.j0 = (tt % tiles_j) * kGT;
    x.i0 = ((tt / tiles_j) % tiles_i) * kGT;
    x.g = tt / (tiles_j * tiles_i);
    const int kb = live ? a.offsets[x.g] : 0;
    x.klen = live ? a.offsets[x.g + 1] - kb : 0;
    x.ar = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.A + (int64_t)kb * a.lda), (short)0,
                                             (int)((int64_t)x.klen * a.lda * 2), 0x00020000);
    x.br = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.B + (int64_t)kb * a.ldb), (short)0,
                                             (int)((int64_t)x.klen * a.ldb * 2), 0x00020000);
    return x;
  };
  bwu32x4_t ra[R][2], rb[R][2];
  auto load = [&](const Tile& x, int st, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[q][h] = __builtin_amdgcn_raw_buffer_load_b128(x.ar, a_off[h], st * a_step + x.i0 * 2, 0);
      rb[q][h] = __builtin_amdgcn_raw_buffer_load_b128(x.br, b_off[h], st * b_step + x.j0 * 2, 0);
    }
  };
  const int ks_off = (8 * (lane >> 4) + 2 * ((lane >> 2) & 3)) * kLdKs + 4 * (lane & 3);
  auto frag = [&](const bf16_t* s, int rowbase) -> bwbf16x8_t {
    const bwv4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_off + rowbase));
    const bwv4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_off + kLdKs + rowbase));
    return __builtin_bit_cast(bwbf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bwf32x4_t acc[4][4];
  // one K step from ring entry q, then refill the entry with step `st` of
  // tile `x`
  auto step = [&](int q, const Tile& x, int st) {
    const int buf = q & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<bwu32x4_t*>(&sA[buf][s_lds[h]]) = ra[q][h];
      *reinterpret_cast<bwu32x4_t*>(&sB[buf][s_lds[h]]) = rb[q][h];
    }
    __syncthreads();
    load(x, st, q);
    bwbf16x8_t fb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = frag(sB[buf], 64 * wc + 16 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bwbf16x8_t fa = frag(sA[buf], 64 * wr + 16 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa, acc[i][j], 0, 0, 0);
    }
  };

  // epilogue constants: this thread's fragment writes start at LDS float
  // acc_lds; its read-outs are rows out_r0 + 16 q of the pass, local column
  // lc, which is tile column 64 (lc / 32) + 32 p + lc % 32
  const int acc_lds = (64 * wr + (lane & 15)) * kCs + 32 * wc + 4 * (lane >> 4);
  const int out_r0 = tid >> 4, out_lc = (tid & 15) * 4;
  const int out_lds = out_r0 * kCs + out_lc;
  const int row_bytes = (int)(a.ldc * 4);
  const int out_voff = out_r0 * row_bytes + (64 * (out_lc >> 5) + (out_lc & 31)) * 4;

  Tile cur = tile_at(t, true);
#pragma unroll
  for (int q = 0; q < R; ++q) load(cur, q, q);
  while (true) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = bwf32x4_t{0.f, 0.f, 0.f, 0.f};
    // the previous tile's epilogue has read its LDS out
    __syncthreads();
    // steps padded to whole rounds of R (at least one: an expert without
    // rows runs one round of zeros and stores a zero gradient)
    const int ns_pad = max(R, (cur.klen + kGK * R - 1) / (kGK * R) * R);
    for (int st0 = 0; st0 < ns_pad - R; st0 += R) {
#pragma unroll
      for (int q = 0; q < R; ++q) step(q, cur, st0 + q + R);
    }
    const int tn = sched.dyn ? sched.at(pos + sched.step) : t + sched.step;
    const bool more = sched.dyn ? tn >= 0 : tn < sched.t_end;
    const Tile nxt = tile_at(more ? tn : t, more);
#pragma unroll
    for (int q = 0; q < R; ++q) step(q, nxt, q);

    // C^T fragments -> LDS -> 128-byte row pieces.  Two passes, each takes
    // the column pieces j = 2p, 2p + 1 of every wave (128 rows x 64 columns,
    // row stride 68 floats: the 16 rows of a fragment write land 4 banks
    // apart), so half of every wave's accumulators is free after the first
    // pass.  Local column lc of pass p is column 64 (lc / 32) + 32 p +
    // lc % 32 of the tile; 8 lanes store one 128-byte line.
    float* sC = reinterpret_cast<float*>(&sAB[0][0]);
    float* Cg = static_cast<float*>(a.C) + (size_t)cur.g * a.c_stride;
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        Cg, (short)0, (int)((int64_t)a.I * a.ldc * 4), 0x00020000);
    // rows left in this tile for the thread's first read-out row; a row past
    // I gets an offset beyond the resource, so its store is dropped
    const int rows_left = a.I - cur.i0 - out_r0;
    const int tile_soff = (int)(((int64_t)cur.i0 * a.ldc + cur.j0) * 4);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          *reinterpret_cast<bwf32x4_t*>(sC + acc_lds + 16 * i * kCs + 16 * jj) = acc[i][2 * p + jj];
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) {   // rows out_r0 + 16 q
        const bwf32x4_t v = *reinterpret_cast<const bwf32x4_t*>(sC + out_lds + 16 * q * kCs);
        const int off = 16 * q < rows_left ? out_voff : (int)0x80000000;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(bwu32x4_t, v), cr, off,
                                               tile_soff + 16 * q * row_bytes + 128 * p, 2 /* nt */);
      }
    }
    if (!more) break;
    t = tn;
    pos += sched.step;
    cur = nxt;
  }
}

// Row-grouped GEMM for experts with many rows (the matrix cores, not the
// weight stream, bound the time): 128 x 256 tiles, each wave 64 x 128 (four
// A and eight B fragments per 32-K step, a quarter fewer LDS bytes per MFMA
// than 64 x 64), a two-step register ring.  A is K-contiguous ([rows][K]);
// B either way, staged as in the 128-wide kernel ([256][32] swizzled, or
// [32][264] read with transposes: 264 keeps the 4-bank row offset of 136).
constexpr int kWideN = 256;
constexpr int kLdKsW = kWideN + 8;
constexpr int kStageW = 32 * kLdKsW;   // 8448 >= 256 * 32
template <bool kBK, int kEpi>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bw_gemm_wide_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][kStageElems];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][kStageW];
  __shared__ int s_g, s_tile, s_x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  if (wave == 0)
    locate_row_tile(a.offsets, a.groups, gridDim.x, blockIdx.x + blockIdx.y * gridDim.x, &s_g, &s_tile, &s_x);
  __syncthreads();
  const int g = s_g;
  if (g < 0) return;
  const int j0 = s_x * kWideN;
  const int64_t row0 = (int64_t)a.offsets[g] + (int64_t)s_tile * kGT;
  const int rows = (int)min((int64_t)kGT, (int64_t)a.offsets[g + 1] - row0);
  const int klen = a.K, ns = (klen + kGK - 1) / kGK;
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(a.A + row0 * a.lda), (short)0, (int)((int64_t)rows * a.lda * 2), 0x00020000);
  const bf16_t* bbase = a.B + (int64_t)g * a.b_stride;
  const int64_t bbytes = kBK ? (int64_t)a.J * a.ldb * 2 : (int64_t)a.K * a.ldb * 2;
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(bbase), (short)0, (int)min(bbytes, (int64_t)0x7FFFFFFF), 0x00020000);
  int a_off[2], a_lds[2], a_kq[2], b_off[4], b_lds[4], b_kq[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 256 * h;
    a_kq[h] = (c & 3) * 8;
    a_off[h] = (int)(((int64_t)(c >> 2) * a.lda + a_kq[h]) * 2);
    a_lds[h] = kc_lds(c >> 2, c & 3);
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int c = tid + 256 * h;
    if (kBK) {
      b_kq[h] = (c & 3) * 8;
      b_off[h] = (int)(((int64_t)(j0 + (c >> 2)) * a.ldb + b_kq[h]) * 2);
      b_lds[h] = kc_lds(c >> 2, c & 3);
    } else {
      b_kq[h] = 0;
      b_off[h] = (int)(((int64_t)(c >> 5) * a.ldb + j0 + (c & 31) * 8) * 2);
      b_lds[h] = ks_row(c >> 5) * kLdKsW + (c & 31) * 8;
    }
  }
  const int b_step = kBK ? kGK * 2 : (int)(kGK * a.ldb * 2);
  constexpr int R = 2;
  const int ns_pad = (ns + R - 1) / R * R;
  bwu32x4_t ra[R][2], rb[R][4];
  auto load = [&](int st, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) ra[q][h] = __builtin_amdgcn_raw_buffer_load_b128(ar, a_off[h], st * kGK * 2, 0);
#pragma unroll
    for (int h = 0; h < 4; ++h) rb[q][h] = __builtin_amdgcn_raw_buffer_load_b128(br, b_off[h], st * b_step, 0);
    // K columns past K of the K-contiguous operands must be zero
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (st * kGK + a_kq[h] >= klen) ra[q][h] = bwu32x4_t{0u, 0u, 0u, 0u};
    if (kBK) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (st * kGK + b_kq[h] >= klen) rb[q][h] = bwu32x4_t{0u, 0u, 0u, 0u};
    }
  };
  bwf32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = bwf32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kc_off = kc_lds(lane & 15, lane >> 4);
  const int ks_offw = (8 * (lane >> 4) + 2 * ((lane >> 2) & 3)) * kLdKsW + 4 * (lane & 3);
  auto step = [&](int q, int next) {
    const int buf = q & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) *reinterpret_cast<bwu32x4_t*>(&sA[buf][a_lds[h]]) = ra[q][h];
#pragma unroll
    for (int h = 0; h < 4; ++h) *reinterpret_cast<bwu32x4_t*>(&sB[buf][b_lds[h]]) = rb[q][h];
    __syncthreads();
    if (next >= 0) load(next, q);
    bwbf16x8_t fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[i] = *reinterpret_cast<const bwbf16x8_t*>(&sA[buf][kc_off + (64 * wr + 16 * i) * kLdKc]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int cb = 128 * wc + 16 * j;
      bwbf16x8_t fb;
      if (kBK) {
        fb = *reinterpret_cast<const bwbf16x8_t*>(&sB[buf][kc_off + cb * kLdKc]);
      } else {
        const bwv4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(&sB[buf][ks_offw + cb]));
        const bwv4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(&sB[buf][ks_offw + kLdKsW + cb]));
        fb = __builtin_bit_cast(bwbf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa[i], acc[i][j], 0, 0, 0);
    }
  };
#pragma unroll
  for (int q = 0; q < R; ++q) load(q, q);
  for (int st0 = 0; st0 < ns_pad - R; st0 += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) step(q, st0 + q + R);
  }
#pragma unroll
  for (int q = 0; q < R; ++q) step(q, -1);
  constexpr bool kNT = kEpi == EPI_F32 ? (MOE_BW_NT & 1) != 0 : (MOE_BW_NT & 4) != 0;
  const bool vec = a.ldc % 4 == 0 && (kEpi < EPI_GELU_BWD || (a.ld_pre % 4 == 0 && a.ld_h % 4 == 0));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ti = 64 * wr + 16 * i + (lane & 15);
      const int c = j0 + 128 * wc + 16 * j + 4 * (lane >> 4);
      if (ti >= rows) continue;
      const int64_t r = row0 + ti;
      if (vec && c + 3 < a.J) {
        epi_store4<kEpi, kNT>(a, a.C, r, c, acc[i][j]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < a.J) epi_store<kEpi>(a, a.C, r, c + e, acc[i][j][e]);
      }
    }
}

// Weight gradients of experts with many rows (matrix-core bound): the
// persistent kernel above on 128 x 256 tiles, each wave 64 x 128 (eight B
// fragments per step), a two-step register ring, B staged as [32][264] for
// the transpose reads; the output leaves in four passes of two column
// pieces per wave.  Needs J a multiple of 256 and ldc == J.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bw_wgrad_wide_kernel(
    GemmArgs a, int tiles_i, int tiles_j, int total) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * kStageElems + 2 * kStageW];
  bf16_t(*sA)[kStageElems] = reinterpret_cast<bf16_t(*)[kStageElems]>(smem);
  bf16_t(*sB)[kStageW] = reinterpret_cast<bf16_t(*)[kStageW]>(smem + 2 * kStageElems);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  constexpr int R = 2;
  constexpr int kCs = 68;   // fp32 LDS row stride of the staged output
  static_assert(128 * kCs * 4 <= (2 * kStageElems + 2 * kStageW) * 2, "staged output fits the stages");
  // this workgroup's tiles: with a grid of whole XCD rounds, a strided walk
  // over its XCD's contiguous range, else over all tiles
  __shared__ int s_list[kMaxExperts];
  WgradSchedule sched;
  sched.list = s_list;
  sched.per_group = tiles_i * tiles_j;
  int t = sched.first(a, total);                   // uniform
  int pos = blockIdx.x / kBwXcds;                  // list position of tile t (plan)
  if (t < 0) return;

  // per thread and step: two 16-byte chunks of each operand, chunk c ->
  // K row c / 16, column offset 8 (c % 16); the tile's first column goes
  // into the scalar offset
  int a_off[2], s_lds[2], b_off[4], sb_lds[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 256 * h;
    const int kr = c >> 4, cc = (c & 15) * 8;
    a_off[h] = (int)(((int64_t)kr * a.lda + cc) * 2);
    s_lds[h] = ks_row(kr) * kLdKs + cc;
  }
  // B: 256 columns, four chunks per thread: K row c / 32, column 8 (c % 32)
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int c = tid + 256 * h;
    const int kr = c >> 5, cc = (c & 31) * 8;
    b_off[h] = (int)(((int64_t)kr * a.ldb + cc) * 2);
    sb_lds[h] = ks_row(kr) * kLdKsW + cc;
  }
  const int a_step = (int)(kGK * a.lda * 2), b_step = (int)(kGK * a.ldb * 2);

  struct Tile {
    __amdgpu_buffer_rsrc_t ar, br;
    int g, i0, j0, klen;
  };
  // tile coordinates and operand resources (rows past the group's K read
  // as zero; `live` false gives empty resources, whose loads return zeros)
  auto tile_at = [&](int tt, bool live) -> Tile {
    Tile x;
    x.j0 = (tt % tiles_j) * kWideN;
    x.i0 = ((tt / tiles_j) % tiles_i) * kGT;
    x.g = tt / (tiles_j * tiles_i);
    const int kb = live ? a.offsets[x.g] : 0;
    x.klen = live ? a.offsets[x.g + 1] - kb : 0;
    x.ar = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.A + (int64_t)kb * a.lda), (short)0,
                                             (int)((int64_t)x.klen * a.lda * 2), 0x00020000);
    x.br = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.B + (int64_t)kb * a.ldb), (short)0,
                                             (int)((int64_t)x.klen * a.ldb * 2), 0x00020000);
    return x;
  };
  bwu32x4_t ra[R][2], rb[R][4];
  auto load = [&](const Tile& x, int st, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ra[q][h] = __builtin_amdgcn_raw_buffer_load_b128(x.ar, a_off[h], st * a_step + x.i0 * 2, 0);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      rb[q][h] = __builtin_amdgcn_raw_buffer_load_b128(x.br, b_off[h], st * b_step + x.j0 * 2, 0);
  };
  const int ks_off = (8 * (lane >> 4) + 2 * ((lane >> 2) & 3)) * kLdKs + 4 * (lane & 3);
  auto frag = [&](const bf16_t* s, int rowbase) -> bwbf16x8_t {
    const bwv4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_off + rowbase));
    const bwv4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_off + kLdKs + rowbase));
    return __builtin_bit_cast(bwbf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  const int ks_offw = (8 * (lane >> 4) + 2 * ((lane >> 2) & 3)) * kLdKsW + 4 * (lane & 3);
  auto fragw = [&](const bf16_t* s, int rowbase) -> bwbf16x8_t {
    const bwv4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_offw + rowbase));
    const bwv4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_v4i16*)(s + ks_offw + kLdKsW + rowbase));
    return __builtin_bit_cast(bwbf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bwf32x4_t acc[4][8];
  // one K step from ring entry q, then refill the entry with step `st` of
  // tile `x`
  auto step = [&](int q, const Tile& x, int st) {
    const int buf = q & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) *reinterpret_cast<bwu32x4_t*>(&sA[buf][s_lds[h]]) = ra[q][h];
#pragma unroll
    for (int h = 0; h < 4; ++h) *reinterpret_cast<bwu32x4_t*>(&sB[buf][sb_lds[h]]) = rb[q][h];
    __syncthreads();
    load(x, st, q);
    bwbf16x8_t fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag(sA[buf], 64 * wr + 16 * i);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bwbf16x8_t fb = fragw(sB[buf], 128 * wc + 16 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa[i], acc[i][j], 0, 0, 0);
    }
  };

  // epilogue constants: this thread's fragment writes start at LDS float
  // acc_lds; its read-outs are rows out_r0 + 16 q of the pass, local column
  // lc, which is tile column 128 (lc / 32) + 32 p + lc % 32
  const int acc_lds = (64 * wr + (lane & 15)) * kCs + 32 * wc + 4 * (lane >> 4);
  const int out_r0 = tid >> 4, out_lc = (tid & 15) * 4;
  const int out_lds = out_r0 * kCs + out_lc;
  const int row_bytes = (int)(a.ldc * 4);
  const int out_voff = out_r0 * row_bytes + (128 * (out_lc >> 5) + (out_lc & 31)) * 4;

  Tile cur = tile_at(t, true);
#pragma unroll
  for (int q = 0; q < R; ++q) load(cur, q, q);
  while (true) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = bwf32x4_t{0.f, 0.f, 0.f, 0.f};
    // the previous tile's epilogue has read its LDS out
    __syncthreads();
    // steps padded to whole rounds of R (at least one: an expert without
    // rows runs one round of zeros and stores a zero gradient)
    const int ns_pad = max(R, (cur.klen + kGK * R - 1) / (kGK * R) * R);
    for (int st0 = 0; st0 < ns_pad - R; st0 += R) {
#pragma unroll
      for (int q = 0; q < R; ++q) step(q, cur, st0 + q + R);
    }
    const int tn = sched.dyn ? sched.at(pos + sched.step) : t + sched.step;
    const bool more = sched.dyn ? tn >= 0 : tn < sched.t_end;
    const Tile nxt = tile_at(more ? tn : t, more);
#pragma unroll
    for (int q = 0; q < R; ++q) step(q, nxt, q);

    // C^T fragments -> LDS -> 128-byte row pieces, four passes of the
    // column pieces j = 2p, 2p + 1 of every wave, as in the 128-wide kernel
    float* sC = reinterpret_cast<float*>(smem);
    float* Cg = static_cast<float*>(a.C) + (size_t)cur.g * a.c_stride;
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        Cg, (short)0, (int)((int64_t)a.I * a.ldc * 4), 0x00020000);
    // rows left in this tile for the thread's first read-out row; a row past
    // I gets an offset beyond the resource, so its store is dropped
    const int rows_left = a.I - cur.i0 - out_r0;
    const int tile_soff = (int)(((int64_t)cur.i0 * a.ldc + cur.j0) * 4);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          *reinterpret_cast<bwf32x4_t*>(sC + acc_lds + 16 * i * kCs + 16 * jj) = acc[i][2 * p + jj];
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) {   // rows out_r0 + 16 q
        const bwf32x4_t v = *reinterpret_cast<const bwf32x4_t*>(sC + out_lds + 16 * q * kCs);
        const int off = 16 * q < rows_left ? out_voff : (int)0x80000000;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(bwu32x4_t, v), cr, off,
                                               tile_soff + 16 * q * row_bytes + 128 * p, 2 /* nt */);
      }
    }
    if (!more) break;
    t = tn;
    pos += sched.step;
    cur = nxt;
  }
}

// Plain grouped GEMM, one thread per output element, fp32 accumulation in
// K order; T = float or bf16.  Same argument meaning as the bf16 kernel.
template <typename T, bool kAK, bool kBK, int kMode, int kEpi>
__global__ __launch_bounds__(256) void bw_gemm_plain_kernel(GemmArgs a, int64_t rows_total) {
  const T* A = reinterpret_cast<const T*>(a.A);
  const T* Bm = reinterpret_cast<const T*>(a.B);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int g;
  int64_t r;
  int c;
  int kbeg = 0, klen = a.K;
  if (kMode == 0) {
    if (idx >= rows_total * a.J) return;
    r = idx / a.J;
    c = (int)(idx % a.J);
    if (r >= a.offsets[a.groups]) return;
    int lo = 0, hi = a.groups - 1;   // last group with offsets[g] <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offsets[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    g = lo;
  } else {
    g = blockIdx.y;
    if (idx >= (int64_t)a.I * a.J) return;
    r = idx / a.J;
    c = (int)(idx % a.J);
    kbeg = a.offsets[g];
    klen = a.offsets[g + 1] - kbeg;
  }
  const T* Bg = kMode == 0 ? Bm + (int64_t)g * a.b_stride : Bm;
  float acc = 0.f;
  for (int kk = 0; kk < klen; ++kk) {
    const int64_t k = kbeg + kk;
    const float av = kAK ? load_f(A + r * a.lda + k) : load_f(A + k * a.lda + r);
    const float bv = kBK ? load_f(Bg + (int64_t)c * a.ldb + (kMode == 0 ? kk : k))
                         : load_f(Bg + (kMode == 0 ? (int64_t)kk : k) * a.ldb + c);
    acc = fmaf(av, bv, acc);
  }
  void* Cg = kMode == 0 ? a.C : (void*)((char*)a.C + (size_t)g * a.c_stride * (kEpi == EPI_F32 ? 4 : sizeof(T)));
  if (kEpi == EPI_F32) {
    static_cast<float*>(Cg)[r * a.ldc + c] = acc;
  } else if (kEpi == EPI_BF16 || kEpi == EPI_BF16_ADD) {
    const T* base = reinterpret_cast<const T*>(a.base);
    const float b = (kEpi == EPI_BF16_ADD && base) ? load_f(base + r * a.ldc + c) : 0.f;
    store_f(static_cast<T*>(Cg) + r * a.ldc + c, b + acc);
  } else {
    const float* pre = a.pre;
    T* h = reinterpret_cast<T*>(a.h_out);
    T* C = static_cast<T*>(Cg);
    if (kEpi == EPI_GELU_BWD) {
      const float x = load_f(pre + r * a.ld_pre + c);
      store_f(C + r * a.ldc + c, acc * gelu_exact_grad(x));
      store_f(h + r * a.ld_h + c, gelu_exact(x));
    } else {
      const float gp = load_f(pre + r * a.ld_pre + c), up = load_f(pre + r * a.ld_pre + a.f + c);
      const float sg = sigm(gp), si = gp * sg;
      store_f(C + r * a.ldc + c, acc * up * (sg * (1.f + gp * (1.f - sg))));
      store_f(C + r * a.ldc + a.f + c, acc * si);
      store_f(h + r * a.ld_h + c, si * up);
    }
  }
}

// Resident workgroups of a persistent kernel per device (CUs x workgroups
// per CU), asked once per kernel (kId) and device; threads that race here
// store the same value.
template <int kId, typename K>
static hipError_t resident_slots(K kernel, int* out) {
  static std::atomic<int> slots_of[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int slots = slots_of[dev].load(std::memory_order_relaxed);
  if (slots == 0) {
    int cus = 0, per_cu = 0;
    const hipError_t e1 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e1 != hipSuccess) return e1;
    const hipError_t e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0);
    if (e2 != hipSuccess) return e2;
    slots = max(1, cus * max(1, per_cu));
    slots_of[dev].store(slots, std::memory_order_relaxed);
  }
  *out = slots;
  return hipSuccess;
}

// Host side: grid and kernel choice.  bf16 on the matrix cores needs the
// K-contiguous operands' leading dimensions to be multiples of 8 (16-byte
// rows), K % 8 == 0, and every leading dimension a multiple of 8; anything
// else, and fp32, runs the plain kernel.
template <bool kAK, bool kBK, int kMode, int kEpi>
static hipError_t run_gemm(const GemmArgs& a, int dtype, int64_t rows_bound, hipStream_t stream) {
  const bool mfma = dtype == 1 && a.lda % 8 == 0 && a.ldb % 8 == 0 && (kMode == 1 || a.K % 8 == 0);
  if (mfma) {
    if constexpr (kMode == 1 && kEpi == EPI_F32 && !kAK && !kBK && MOE_BW_PERSIST) {
      // (rows up to a tile past I keep every store offset below 2^31)
      if (a.J % kGT == 0 && a.ldc == a.J && ((int64_t)a.I + kGT) * a.ldc * 4 <= INT32_MAX) {
        const bool wide = MOE_BW_WIDE && a.J % kWideN == 0 && rows_bound >= (int64_t)MOE_BW_WIDE_ROWS * a.groups;
        int slots = 0;
        const hipError_t es = wide ? resident_slots<1>(bw_wgrad_wide_kernel, &slots)
                                   : resident_slots<0>(bw_wgrad_bf16_kernel, &slots);
        if (es != hipSuccess) return es;
        const int ti = (a.I + kGT - 1) / kGT, tj = a.J / (wide ? kWideN : kGT);
        const int64_t total = (int64_t)ti * tj * a.groups;
        if (total == 0) return hipSuccess;
        int grid = (int)(total < slots ? total : (int64_t)slots);
        // a plan needs every XCD to hold a workgroup: whole rounds of 8
        // (without them the kernels fall back to the equal split)
        if (grid >= kBwXcds) grid -= grid % kBwXcds;
        const GemmArgs& ap = a;
        if (wide)
          hipLaunchKernelGGL(bw_wgrad_wide_kernel, dim3((unsigned)grid), dim3(256), 0, stream, ap, ti, tj, (int)total);
        else
          hipLaunchKernelGGL(bw_wgrad_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, ap, ti, tj, (int)total);
        return hipGetLastError();
      }
    }
    // many rows per expert (past the matrix-core ridge): the wide tiles
    if constexpr (kMode == 0 && kAK && kEpi != EPI_BF16_ADD && kEpi != EPI_GELU_BWD) {
      if (MOE_BW_WIDE && a.J % kWideN == 0 && rows_bound >= (int64_t)MOE_BW_WIDE_ROWS * a.groups) {
        const dim3 grid((unsigned)(a.J / kWideN), (unsigned)((rows_bound + kGT - 1) / kGT + a.groups), 1);
        hipLaunchKernelGGL((bw_gemm_wide_kernel<kBK, kEpi>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
      }
    }
    dim3 grid;
    if (kMode == 0)
      grid = dim3((unsigned)((a.J + kGT - 1) / kGT), (unsigned)((rows_bound + kGT - 1) / kGT + a.groups), 1);
    else
      grid = dim3((unsigned)((a.J + kGT - 1) / kGT), (unsigned)((a.I + kGT - 1) / kGT), (unsigned)a.groups);
    hipLaunchKernelGGL((bw_gemm_bf16_kernel<kAK, kBK, kMode, kEpi>), grid, dim3(256), 0, stream, a);
  } else {
    if (kMode == 0) {
      const int64_t total = rows_bound * a.J;
      if (total == 0) return hipSuccess;
      const dim3 grid((unsigned)((total + 255) / 256));
      if (dtype == 1)
        hipLaunchKernelGGL((bw_gemm_plain_kernel<bf16_t, kAK, kBK, kMode, kEpi>), grid, dim3(256), 0, stream, a,
                           rows_bound);
      else
        hipLaunchKernelGGL((bw_gemm_plain_kernel<float, kAK, kBK, kMode, kEpi>), grid, dim3(256), 0, stream, a,
                           rows_bound);
    } else {
      const dim3 grid((unsigned)(((int64_t)a.I * a.J + 255) / 256), (unsigned)a.groups);
      if (dtype == 1)
        hipLaunchKernelGGL((bw_gemm_plain_kernel<bf16_t, kAK, kBK, kMode, kEpi>), grid, dim3(256), 0, stream, a,
                           (int64_t)0);
      else
        hipLaunchKernelGGL((bw_gemm_plain_kernel<float, kAK, kBK, kMode, kEpi>), grid, dim3(256), 0, stream, a,
                           (int64_t)0);
    }
  }
  return hipGetLastError();
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: the pre-activation in fp32 (it feeds act' and act, so it is
// not rounded to bf16), H and dA in the activation type, then the weight
// gradients' schedule (wgrad_plan_kernel: 8 E + 8 int32).
static size_t plan_bytes(int E) { return al256(((size_t)8 * E + 8) * 4); }
size_t ffn_backward_workspace_bytes(int64_t M_max, int E, int d, int f, int act, int dtype) {
  (void)d;
  const size_t eb = dtype == 1 ? 2 : 4;
  const int64_t fr = act == 1 ? 2 * (int64_t)f : f;
  const int64_t M = M_max > 0 ? M_max : 0;
  return al256((size_t)M * fr * 4) + al256((size_t)M * f * eb) + al256((size_t)M * fr * eb) + plan_bytes(E);
}

hipError_t launch_expert_ffn_backward(const void* X_perm, int dtype, const int32_t* expert_offset, int E, int d,
                                      int f, int act, const void* W1, const void* W2, const void* dY_perm,
                                      int64_t M_max, void* dX_perm, float* dW1, float* dW2, void* ws,
                                      hipStream_t stream) {
  const size_t eb = dtype == 1 ? 2 : 4;
  const int fr = act == 1 ? 2 * f : f;
  const int64_t M = M_max > 0 ? M_max : 0;
  char* w = static_cast<char*>(ws);
  float* pre = reinterpret_cast<float*>(w);
  void* h = w + al256((size_t)M * fr * 4);
  void* da = w + al256((size_t)M * fr * 4) + al256((size_t)M * f * eb);
  int32_t* plan = reinterpret_cast<int32_t*>(static_cast<char*>(da) + al256((size_t)M * fr * eb));
  hipError_t err;
  // 1 + 2 fused (GELU on the matrix cores): dA, H straight from both products
  const bool fuse = MOE_BW_FUSE_DH && act == 0 && dtype == 1 && d % 8 == 0 && f % 8 == 0;
  if (fuse) {
    GemmArgs a{};
    a.A = static_cast<const bf16_t*>(dY_perm);
    a.lda = d;
    a.B = static_cast<const bf16_t*>(W2);
    a.ldb = f;
    a.b_stride = (int64_t)d * f;
    a.C = da;
    a.ldc = fr;
    a.offsets = expert_offset;
    a.groups = E;
    a.J = f;
    a.K = d;
    a.h_out = static_cast<bf16_t*>(h);
    a.ld_h = f;
    a.f = f;
    const dim3 grid((unsigned)((f + kGT - 1) / kGT), (unsigned)((M + kGT - 1) / kGT + E), 1);
    hipLaunchKernelGGL(bw_dh_gelu_fused_kernel, grid, dim3(256), 0, stream, a, static_cast<const bf16_t*>(X_perm),
                       static_cast<const bf16_t*>(W1));
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 1. pre-activation A = X W1^T  (row-grouped; W1[e] is [fr][d]: K-contiguous)
  if (!fuse) {
    GemmArgs a{};
    a.A = static_cast<const bf16_t*>(X_perm);
    a.lda = d;
    a.B = static_cast<const bf16_t*>(W1);
    a.ldb = d;
    a.b_stride = (int64_t)fr * d;
    a.C = pre;
    a.ldc = fr;
    a.offsets = expert_offset;
    a.groups = E;
    a.J = fr;
    a.K = d;
    // bf16 with d and f_rows multiples of 64 (the shapes the forward's
    // kernel serves: whole 16-byte pieces of every output row): its
    // LDS-tiled grouped GEMM (32x32x16 products, 64-wide K stages) with an
    // fp32 epilogue
    err = dtype == 1 && d % 64 == 0 && fr % 64 == 0 && M > 0
              ? launch_rows_gemm_f32(X_perm, expert_offset, E, W1, fr, d, M, pre, stream)
              : run_gemm<true, true, 0, EPI_F32>(a, dtype, M, stream);
    if (err != hipSuccess) return err;
  }
  // 2. dH = dY W2 with the activation backward in the epilogue: dA, H
  //    (W2[e] is [d][f]: K = d is its row index)
  if (!fuse) {
    GemmArgs a{};
    a.A = static_cast<const bf16_t*>(dY_perm);
    a.lda = d;
    a.B = static_cast<const bf16_t*>(W2);
    a.ldb = f;
    a.b_stride = (int64_t)d * f;
    a.C = da;
    a.ldc = fr;
    a.offsets = expert_offset;
    a.groups = E;
    a.J = f;
    a.K = d;
    a.pre = pre;
    a.ld_pre = fr;
    a.h_out = static_cast<bf16_t*>(h);
    a.ld_h = f;
    a.f = f;
    err = act == 1 ? run_gemm<true, false, 0, EPI_SWIGLU_BWD>(a, dtype, M, stream)
                   : run_gemm<true, false, 0, EPI_GELU_BWD>(a, dtype, M, stream);
    if (err != hipSuccess) return err;
  }
  // 3. dX = dA W1 (W1[e] is [fr][d]: K = fr is its row index)
  {
    GemmArgs a{};
    a.A = static_cast<const bf16_t*>(da);
    a.lda = fr;
    a.B = static_cast<const bf16_t*>(W1);
    a.ldb = d;
    a.b_stride = (int64_t)fr * d;
    a.C = dX_perm;
    a.ldc = d;
    a.offsets = expert_offset;
    a.groups = E;
    a.J = d;
    a.K = fr;
    // bf16 with f_rows and d multiples of 64 and experts averaging fewer rows
    // than the wide tiles take: the forward's LDS-tiled grouped GEMM reading
    // W1 K-major through transposing LDS reads (expert choice: 294 -> 242
    // us; with many rows per expert the wide kernel measured 8% faster)
    err = dtype == 1 && fr % 64 == 0 && d % 64 == 0 && M > 0 && M < (int64_t)MOE_BW_WIDE_ROWS * E
              ? launch_rows_gemm_kmajor(da, expert_offset, E, W1, d, fr, M, dX_perm, stream)
              : run_gemm<true, false, 0, EPI_BF16>(a, dtype, M, stream);
    if (err != hipSuccess) return err;
  }
  // 4. dW2[e] = dY^T H  (K-grouped over the expert's rows), after the
  //    weight gradients' schedule
  hipLaunchKernelGGL(wgrad_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, expert_offset, E, plan);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    GemmArgs a{};
    a.plan = plan;
    a.A = static_cast<const bf16_t*>(dY_perm);
    a.lda = d;
    a.B = static_cast<const bf16_t*>(h);
    a.ldb = f;
    a.C = dW2;
    a.ldc = f;
    a.c_stride = (int64_t)d * f;
    a.offsets = expert_offset;
    a.groups = E;
    a.I = d;
    a.J = f;
    err = run_gemm<false, false, 1, EPI_F32>(a, dtype, M, stream);
    if (err != hipSuccess) return err;
  }
  // 5. dW1[e] = dA^T X
  {
    GemmArgs a{};
    a.plan = plan;
    a.A = static_cast<const bf16_t*>(da);
    a.lda = fr;
    a.B = static_cast<const bf16_t*>(X_perm);
    a.ldb = d;
    a.C = dW1;
    a.ldc = d;
    a.c_stride = (int64_t)fr * d;
    a.offsets = expert_offset;
    a.groups = E;
    a.I = fr;
    a.J = d;
    err = run_gemm<false, false, 1, EPI_F32>(a, dtype, M, stream);
  }
  return err;
}

// Router backward: dX = base + dZ W_g^T, dW_g = X^T dZ (K split into
// kRouterBwSplits slices of rows summed in slice order), d_offset = column
// sums of dZ.  dZ is first rounded to the activation type (the matrix-core
// operand); the workspace holds it, the slice partials and two offset
// tables ({0, n} and the slice bounds).
constexpr int kRouterBwSplits = 16;

size_t router_backward_workspace_bytes(int n, int d, int E, int dtype) {
  const size_t eb = dtype == 1 ? 2 : 4;
  return al256((size_t)n * E * eb) + al256((size_t)kRouterBwSplits * d * E * 4) +
         al256((size_t)(kRouterBwSplits + 3) * sizeof(int32_t));
}

__global__ __launch_bounds__(256) void to_dtype_kernel(const float* __restrict__ src, int64_t count, int dtype,
                                                       void* __restrict__ dst, int32_t* __restrict__ offs,
                                                       int n, int splits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) {
    if (dtype == 1) static_cast<bf16_t*>(dst)[i] = f32_to_bf16(src[i]);
    else static_cast<float*>(dst)[i] = src[i];
  }
  // offs[0..1] = {0, n}; offs[2 .. 2 + splits] = slice bounds
  if (i < 2) offs[i] = i == 0 ? 0 : n;
  if (i <= splits) offs[2 + i] = (int32_t)(((int64_t)n * i) / splits);
}

__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int64_t count, int splits,
                                                        float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float v = part[i];
  for (int s = 1; s < splits; ++s) v = v + part[(int64_t)s * count + i];
  out[i] = v;
}

// One workgroup per expert: thread i adds rows i, i + 256, ... in order,
// then a halving tree over the 256 partial sums.
__global__ __launch_bounds__(256) void col_sum_kernel(const float* __restrict__ dz, int n, int E,
                                                      float* __restrict__ out) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float v = 0.f;
  for (int t = threadIdx.x; t < n; t += 256) v = v + dz[(size_t)t * E + e];
  red[threadIdx.x] = v;
  for (int s = 128; s >= 1; s >>= 1) {
    __syncthreads();
    if ((int)threadIdx.x < s) red[threadIdx.x] = red[threadIdx.x] + red[threadIdx.x + s];
  }
  if (threadIdx.x == 0) out[e] = red[0];
}

hipError_t launch_router_backward(const void* X, const void* Wg, int dtype, const float* dZ, int n, int d, int E,
                                  const void* base, void* dX, float* dWg, float* d_offset, void* ws,
                                  hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const size_t eb = dtype == 1 ? 2 : 4;
  char* w = static_cast<char*>(ws);
  void* dz_t = w;
  float* part = reinterpret_cast<float*>(w + al256((size_t)n * E * eb));
  int32_t* offs =
      reinterpret_cast<int32_t*>(w + al256((size_t)n * E * eb) + al256((size_t)kRouterBwSplits * d * E * 4));
  const int64_t cnt = (int64_t)n * E;
  hipLaunchKernelGGL(to_dtype_kernel, dim3((unsigned)((max(cnt, (int64_t)kRouterBwSplits + 1) + 255) / 256)),
                     dim3(256), 0, stream, dZ, cnt, dtype, dz_t, offs, n, kRouterBwSplits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dX) {
    // one group of n rows; W_g [d][E] is K-contiguous along E
    GemmArgs a{};
    a.A = static_cast<const bf16_t*>(dz_t);
    a.lda = E;
    a.B = static_cast<const bf16_t*>(Wg);
    a.ldb = E;
    a.C = dX;
    a.ldc = d;
    a.offsets = offs;
    a.groups = 1;
    a.J = d;
    a.K = E;
    a.base = static_cast<const bf16_t*>(base);
    err = run_gemm<true, true, 0, EPI_BF16_ADD>(a, dtype, n, stream);
    if (err != hipSuccess) return err;
  }
  if (dWg) {
    GemmArgs a{};
    a.A = static_cast<const bf16_t*>(X);
    a.lda = d;
    a.B = static_cast<const bf16_t*>(dz_t);
    a.ldb = E;
    a.C = part;
    a.ldc = E;
    a.c_stride = (int64_t)d * E;
    a.offsets = offs + 2;
    a.groups = kRouterBwSplits;
    a.I = d;
    a.J = E;
    err = run_gemm<false, false, 1, EPI_F32>(a, dtype, 0, stream);
    if (err != hipSuccess) return err;
    const int64_t c2 = (int64_t)d * E;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((c2 + 255) / 256)), dim3(256), 0, stream, part, c2,
                       kRouterBwSplits, dWg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (d_offset) {
    hipLaunchKernelGGL(col_sum_kernel, dim3((unsigned)E), dim3(256), 0, stream, dZ, n, E, d_offset);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
