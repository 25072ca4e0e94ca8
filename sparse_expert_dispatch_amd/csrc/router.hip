// Router: Z = X W_g (+ per-expert offset), then the specified score
// transform (softmax over experts, or a sigmoid per expert).
//
// MoE-routing pages: page 2 "Expert choice routing", section "The math"
// (S = softmax(X W_g), X: [n, d], W_g: [d, E]); page 5 "MoE routing
// strategies explained", strategy 4 (sigmoid scores).
//
// bf16 path, two kernels: the GEMM kernel runs v_mfma_f32_16x16x32_bf16 on
// 128-row x 64-expert workgroup tiles, X read once from HBM; each K stage of
// W_g [d, E] is loaded once per workgroup and transposed on its way into
// LDS ([expert][K] rows, so a matrix-core B fragment is one 16-byte read);
// K is split across workgroups (up to 8 slices) until the grid fills the
// GPU.  The per-slice partial logits go to the workspace; the
// finalize kernel adds the slices in slice order (so the result is
// deterministic), adds the offset and evaluates the scores.

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRouterBK = 64;      // K per pipeline stage
constexpr int kRouterSplitsMax = 8;

// Z = X W_g on the matrix cores.  A workgroup (4 waves) owns 128 token rows
// and 64 expert columns over one K slice: each wave 32 rows (2 x 4 tiles of
// v_mfma_f32_16x16x32_bf16), its X fragments loaded straight from HBM as
// 16-byte chunks of 8 consecutive K values; the 64 x 64 W_g^T block of each
// K stage is loaded once per workgroup into LDS (rows padded by 16 bytes:
// the fragment reads are conflict-free) and shared by the four waves.  With
// 16 rows per wave and W_g^T fragments read from L2 by every wave, W_g
// traffic was four times X's; here it is half.  The next stage's X and W_g^T
// loads are in flight in registers while the current stage is multiplied.
constexpr int kRouterRows = 128;   // token rows per workgroup (4 waves x 32)
constexpr int kRouterAhead = 4;    // K stages in flight
constexpr int kRouterECols = 64;   // expert columns per workgroup
constexpr int kRouterWStride = kRouterBK + 8;

__global__ __launch_bounds__(256) void router_gemm_bf16_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ Wg, int n, int d, int E, int k_per_split,
    float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) bf16_t sW[2][kRouterECols * kRouterWStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blockIdx.x * kRouterRows + 32 * wave;
  const int c0 = blockIdx.z * kRouterECols;
  const int split = blockIdx.y;
  const int nt = min(4, (E - c0) >> 4);                 // 16-column tiles of this workgroup
  const int kbeg = split * k_per_split;
  const int nk = k_per_split / kRouterBK;
  const int kl = (lane >> 4) << 3;
  // X fragment sources: row tile i, lane -> row (lane % 16), K offset kl
  const bf16_t* xp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) xp[i] = X + (size_t)min(row0 + 16 * i + (lane & 15), n - 1) * d + kbeg + kl;
  // W_g stage loads straight from the [d, E] layout: 64 K rows x 8 chunks of
  // 8 experts, two chunks per thread (experts past E re-read the last
  // chunk; their columns are never stored); the LDS store transposes them
  // into [expert][K] rows
  const int wk = tid >> 3, we = (tid & 7) << 3;
  const bf16_t* wp[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) wp[h] = Wg + (size_t)(kbeg + wk + 32 * h) * E + min(c0 + we, E - 8);

  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Stage ring: kRouterAhead stages of X (registers) and W_g^T (registers,
  // then LDS) are in flight while the oldest is multiplied; ring slots are
  // compile-time (a partial last round is skipped stage by stage, uniformly
  // across the workgroup).
  bf16x8_t xr[kRouterAhead][2][2];                      // [slot][32-wide K step][row tile]
  u32x4_t wr_[kRouterAhead][2];
  auto load = [&](int st, int q) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) xr[q][s][i] = *reinterpret_cast<const bf16x8_t*>(xp[i] + st * kRouterBK + 32 * s);
#pragma unroll
    for (int h = 0; h < 2; ++h) wr_[q][h] = *reinterpret_cast<const u32x4_t*>(wp[h] + (size_t)st * kRouterBK * E);
  };
  auto store_w = [&](int q, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16_t* v = reinterpret_cast<const bf16_t*>(&wr_[q][h]);
#pragma unroll
      for (int j = 0; j < 8; ++j) sW[buf][(we + j) * kRouterWStride + wk + 32 * h] = v[j];
    }
  };
#pragma unroll
  for (int q = 0; q < kRouterAhead; ++q)
    if (q < nk) load(q, q);
  for (int st0 = 0; st0 < nk; st0 += kRouterAhead) {
#pragma unroll
    for (int q = 0; q < kRouterAhead; ++q) {
      const int st = st0 + q;
      if (st >= nk) break;
      const int buf = st & 1;
      store_w(q, buf);
      __syncthreads();                               // W stage visible; the other buffer is free
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < nt) {
            const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(
                &sW[buf][(16 * j + (lane & 15)) * kRouterWStride + 32 * s + kl]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[q][s][i], b, acc[i][j], 0, 0, 0);
          }
        }
      }
      if (st + kRouterAhead < nk) load(st + kRouterAhead, q);
    }
  }
  // C fragment: lane holds column (lane % 16), rows (lane / 16) * 4 + r.
  float* out = partial + (size_t)split * n * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nt) {
        const int col = c0 + j * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row0 + 16 * i + ((lane >> 4) << 2) + r;
          if (row < n) out[(size_t)row * E + col] = acc[i][j][r];
        }
      }
    }
}

// Scalar router for fp32 inputs and for shapes the MFMA tiling does not
// cover: one thread per (row, expert), sequential fp32 FMA over d.
MOE_DEV float load_elem(const float* p) { return *p; }
MOE_DEV float load_elem(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__global__ __launch_bounds__(256) void router_gemm_scalar_kernel(const T* __restrict__ X,
                                                                 const T* __restrict__ Wg, int n,
                                                                 int d, int E, float* __restrict__ z) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n * E) return;
  const int row = (int)(i / E), e = (int)(i - (int64_t)row * E);
  const T* x = X + (size_t)row * d;
  float acc = 0.f;
  for (int kk = 0; kk < d; ++kk) acc = fmaf(load_elem(x + kk), load_elem(Wg + (size_t)kk * E + e), acc);
  z[i] = acc;
}

static bool router_uses_mfma(int dtype, int d, int E) { return dtype == 1 && d % 64 == 0 && E % 16 == 0; }

// Finalize: 16 rows per workgroup, one wave per row at a time; lane l holds
// experts l + 64 j.  Sums the split partials in split order, adds the
// offset, then the scaled noise of noisy top-k (page 4 "How MoE routing
// strategies ...", section "Pitfalls": Gaussian noise on the gating
// logits; the standard normals are an input), writes the logits and (on
// request) the specified scores,
// row-major and/or transposed.  The transpose goes through an LDS tile with
// an odd row stride (E + 1 floats), so both the row-wise writes and the
// column-wise reads are free of bank conflicts and the [E, n] stores are
// 64-byte runs.
constexpr int kFinRows = 16;

__global__ __launch_bounds__(1024) void router_finalize_kernel(
    const float* partial, int nsplit, int n, int E, const float* __restrict__ offset,
    const float* __restrict__ noise, float noise_std, int score, float* logits,
    float* __restrict__ scores, float* __restrict__ scores_t) {
  // `partial` and `logits` may be the same buffer (single K-slice): each
  // element is read and then written by the same thread.
#pragma clang fp contract(off)
  extern __shared__ float sT[];   // [kFinRows][E + 1] when scores_t is requested
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nj = (E + 63) >> 6;
  const int P = next_pow2(E);
  const int ld = E + 1;
  const int blk_row0 = blockIdx.x * kFinRows;
  for (int rr = wave; rr < kFinRows; rr += 16) {
    const int row = blk_row0 + rr;
    if (row >= n) break;
    float z[kMaxExpertRegs];
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) {
      const int e = lane + 64 * j;
      z[j] = 0.f;
      if (j < nj && e < E) {
        // all slices' loads in flight at once, then added in slice order
        float ps[kRouterSplitsMax];
#pragma unroll
        for (int s = 0; s < kRouterSplitsMax; ++s)
          ps[s] = s < nsplit ? partial[(size_t)s * n * E + (size_t)row * E + e] : 0.f;
        float v = ps[0];
#pragma unroll
        for (int s = 1; s < kRouterSplitsMax; ++s)
          if (s < nsplit) v = v + ps[s];
        if (offset) v = v + offset[e];
        if (noise) v = v + noise_std * noise[(size_t)row * E + e];
        z[j] = v;
        if (logits) logits[(size_t)row * E + e] = v;
      }
    }
    if (!scores && !scores_t) continue;
    float p[kMaxExpertRegs];
    if (score == 0) {   // softmax
      float m = -__builtin_huge_valf();
#pragma unroll
      for (int j = 0; j < kMaxExpertRegs; ++j)
        if (j < nj && lane + 64 * j < E) m = fmaxf(m, z[j]);
      m = wave_max_f32(m);
      float t[kMaxExpertRegs];
#pragma unroll
      for (int j = 0; j < kMaxExpertRegs; ++j)
        t[j] = (j < nj && lane + 64 * j < E) ? spec_exp(z[j] - m) : 0.f;
      const float s = row_tree_sum(t, P);
#pragma unroll
      for (int j = 0; j < kMaxExpertRegs; ++j) p[j] = t[j] / s;
    } else {
#pragma unroll
      for (int j = 0; j < kMaxExpertRegs; ++j) p[j] = spec_expert_score(z[j], score);
    }
#pragma unroll
    for (int j = 0; j < kMaxExpertRegs; ++j) {
      const int e = lane + 64 * j;
      if (j < nj && e < E) {
        if (scores) scores[(size_t)row * E + e] = p[j];
        if (scores_t) sT[rr * ld + e] = p[j];
      }
    }
  }
  if (!scores_t) return;
  __syncthreads();
  const int rows = min(kFinRows, n - blk_row0);
  for (int item = threadIdx.x; item < E * kFinRows; item += 1024) {
    const int e = item / kFinRows, rr = item % kFinRows;
    if (rr < rows) scores_t[(size_t)e * n + blk_row0 + rr] = sT[rr * ld + e];
  }
}

// ------------------------------------------------------------------ host side

hipError_t launch_router_finalize(const float* partial, int nsplit, int n, int E, const float* offset,
                                  const float* noise, float noise_std, int score, float* logits,
                                  float* scores, float* scores_t, hipStream_t stream);

static int router_row_blocks(int n) { return (n + kRouterRows - 1) / kRouterRows; }

// Split K until there are at least MOE_ROUTER_MIN_WGS workgroups (each
// slice a multiple of the 64-wide stage).
#ifndef MOE_ROUTER_MIN_WGS
#define MOE_ROUTER_MIN_WGS 256
#endif
static int router_splits(int n, int d, int E) {
  const int blocks = router_row_blocks(n) * ((E + kRouterECols - 1) / kRouterECols);
  const int kb = d / kRouterBK;
  int s = 1;
  while (s < kRouterSplitsMax && blocks * s < MOE_ROUTER_MIN_WGS && kb % (2 * s) == 0) s *= 2;
  return s;
}

size_t router_workspace_bytes(int n, int d, int E, int dtype) {
  if (!router_uses_mfma(dtype, d, E)) return 0;
  const int s = router_splits(n, d, E);
  return s > 1 ? (size_t)s * n * E * sizeof(float) : 0;
}

hipError_t launch_router(const void* X, const void* Wg, int dtype, const float* offset,
                         const float* noise, float noise_std, int n, int d, int E, int score,
                         float* logits, float* scores, float* scores_t, void* ws, hipStream_t stream) {
  const float* partial = logits;
  int nsplit = 1;
  const int64_t total = (int64_t)n * E;
  const dim3 sgrid((unsigned)((total + 255) / 256));
  if (router_uses_mfma(dtype, d, E)) {
    nsplit = router_splits(n, d, E);
    float* dst = nsplit > 1 ? static_cast<float*>(ws) : logits;
    dim3 grid(router_row_blocks(n), nsplit, (E + kRouterECols - 1) / kRouterECols);
    hipLaunchKernelGGL(router_gemm_bf16_kernel, grid, dim3(256), 0, stream,
                       static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(Wg), n, d, E, d / nsplit, dst);
    partial = dst;
  } else if (dtype == 1) {
    hipLaunchKernelGGL(router_gemm_scalar_kernel<bf16_t>, sgrid, dim3(256), 0, stream,
                       static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(Wg), n, d, E, logits);
  } else {
    hipLaunchKernelGGL(router_gemm_scalar_kernel<float>, sgrid, dim3(256), 0, stream,
                       static_cast<const float*>(X), static_cast<const float*>(Wg), n, d, E, logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_router_finalize(partial, nsplit, n, E, offset, noise, noise_std, score, logits, scores,
                                scores_t, stream);
}

hipError_t launch_router_finalize(const float* partial, int nsplit, int n, int E, const float* offset,
                                  const float* noise, float noise_std, int score, float* logits,
                                  float* scores, float* scores_t, hipStream_t stream) {
  const size_t lds = scores_t ? (size_t)kFinRows * (E + 1) * sizeof(float) : 0;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_finalize_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(router_finalize_kernel, dim3((n + kFinRows - 1) / kFinRows), dim3(1024), lds, stream, partial,
                     nsplit, n, E, offset, noise, noise_std, score, logits, scores, scores_t);
  return hipGetLastError();
}

}  // namespace moe
