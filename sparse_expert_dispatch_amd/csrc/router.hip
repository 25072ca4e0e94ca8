// Router: Z = X W_g (+ per-expert offset), then the specified score
// transform (softmax over experts, or a sigmoid per expert).
//
// MoE-routing pages: page 2 "Expert choice routing", section "The math"
// (S = softmax(X W_g), X: [n, d], W_g: [d, E]); page 5 "MoE routing
// strategies explained", strategy 4 (sigmoid scores).
//
// bf16 path: one workgroup = 4 waves = 64 token rows x up to 256 experts,
// over one K-slice of d (split-K when n alone gives too few workgroups to
// fill 256 CUs).  A wave owns 16 rows; its A fragments come straight from
// HBM (X is read exactly once), the W_g slice is staged through LDS
// transposed to [E][K] so every lane reads its 8 consecutive K values of a
// column with one 16-byte LDS read, and the products run on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Per-slice partial logits
// go to a workspace; the finalize kernel adds the slices in slice order (so
// the result is deterministic), adds the offset and evaluates the scores.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRouterRows = 64;    // rows per workgroup (16 per wave)
constexpr int kRouterBK = 64;      // K per LDS stage
constexpr int kRouterCols = 256;   // expert columns per workgroup
constexpr int kRouterLdsStride = kRouterBK + 8;   // bf16 elements per LDS row (padding skews banks)
constexpr int kRouterMaxItems = kRouterBK * kRouterCols / 8 / 256;   // 16-byte W_g loads per thread

// Software pipeline: while the matrix cores work on K stage s (A fragments
// in registers, the W_g stage in LDS buffer s % 2), the next stage's A
// fragments and W_g rows are already loading into registers; they are
// written (transposed) to the other LDS buffer after the MFMAs, so one
// barrier per stage suffices.
__global__ __launch_bounds__(256) void router_gemm_bf16_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ Wg, int n, int d, int E, int k_per_split,
    float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][kRouterCols * kRouterLdsStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = blockIdx.x * kRouterRows + wave * 16;
  const int split = blockIdx.y;
  const int c0 = blockIdx.z * kRouterCols;
  const int ncols = min(kRouterCols, E - c0);     // multiple of 16
  const int nt = ncols >> 4;                       // 16-column tiles
  const int kbeg = split * k_per_split;
  const int nk = k_per_split / kRouterBK;
  const int per_row = ncols >> 3;                  // 8-column chunks per K row
  const int items = kRouterBK * per_row;

  f32x4_t acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A fragment source: row (lane % 16), 8 K values at (lane / 16) * 8.
  int arow = row0 + (lane & 15);
  if (arow > n - 1) arow = n - 1;                  // tail rows are computed but never stored
  const bf16_t* aptr = X + (size_t)arow * d + kbeg + ((lane >> 4) << 3);

  u32x4_t wreg[kRouterMaxItems];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kRouterMaxItems; ++i) {
      const int item = tid + 256 * i;
      if (item < items) {
        const int kk = item / per_row;
        const int cc = (item - kk * per_row) << 3;
        wreg[i] = *reinterpret_cast<const u32x4_t*>(Wg + (size_t)(k0 + kk) * E + c0 + cc);
      }
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kRouterMaxItems; ++i) {
      const int item = tid + 256 * i;
      if (item < items) {
        const int kk = item / per_row;
        const int cc = (item - kk * per_row) << 3;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          sB[buf][(cc + 2 * h) * kRouterLdsStride + kk] = (bf16_t)(wreg[i][h] & 0xFFFFu);
          sB[buf][(cc + 2 * h + 1) * kRouterLdsStride + kk] = (bf16_t)(wreg[i][h] >> 16);
        }
      }
    }
  };

  load_w(kbeg);
  bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(aptr);
  bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(aptr + 32);
  store_w(0);
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nk;
    bf16x8_t na0 = a0, na1 = a1;
    if (more) {
      load_w(kbeg + (s + 1) * kRouterBK);
      na0 = *reinterpret_cast<const bf16x8_t*>(aptr + (s + 1) * kRouterBK);
      na1 = *reinterpret_cast<const bf16x8_t*>(aptr + (s + 1) * kRouterBK + 32);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < nt) {
        const bf16_t* bp = sB[cur] + (j * 16 + (lane & 15)) * kRouterLdsStride + ((lane >> 4) << 3);
        bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(bp);
        bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(bp + 32);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[j], 0, 0, 0);
      }
    }
    if (more) store_w(cur ^ 1);
    a0 = na0;
    a1 = na1;
  }
  // C fragment: lane holds column (lane % 16), rows (lane / 16) * 4 + r.
  float* out = partial + (size_t)split * n * E;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < nt) {
      const int col = c0 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + ((lane >> 4) << 2) + r;
        if (row < n) out[(size_t)row * E + col] = acc[j][r];
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
// offset, writes the logits and (on request) the specified scores,
// row-major and/or transposed.  The transpose goes through an LDS tile with
// an odd row stride (E + 1 floats), so both the row-wise writes and the
// column-wise reads are free of bank conflicts and the [E, n] stores are
// 64-byte runs.
constexpr int kFinRows = 16;

__global__ __launch_bounds__(1024) void router_finalize_kernel(
    const float* partial, int nsplit, int n, int E, const float* __restrict__ offset, int score,
    float* logits, float* __restrict__ scores, float* __restrict__ scores_t) {
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
        float v = partial[(size_t)row * E + e];
        for (int s = 1; s < nsplit; ++s) v = v + partial[(size_t)s * n * E + (size_t)row * E + e];
        if (offset) v = v + offset[e];
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
      for (int j = 0; j < kMaxExpertRegs; ++j) p[j] = spec_sigmoid(z[j]);
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
                                  int score, float* logits, float* scores, float* scores_t,
                                  hipStream_t stream);

static int router_splits(int n, int d) {
  const int row_blocks = (n + kRouterRows - 1) / kRouterRows;
  const int kb = d / kRouterBK;
  int s = 1;
  while (s < 4 && row_blocks * s < 256 && kb % (2 * s) == 0) s *= 2;
  return s;
}

size_t router_workspace_bytes(int n, int d, int E, int dtype) {
  if (!router_uses_mfma(dtype, d, E)) return 0;
  const int s = router_splits(n, d);
  return s > 1 ? (size_t)s * n * E * sizeof(float) : 0;
}

hipError_t launch_router(const void* X, const void* Wg, int dtype, const float* offset, int n, int d,
                         int E, int score, float* logits, float* scores, float* scores_t, void* ws,
                         hipStream_t stream) {
  const float* partial = logits;
  int nsplit = 1;
  const int64_t total = (int64_t)n * E;
  const dim3 sgrid((unsigned)((total + 255) / 256));
  if (router_uses_mfma(dtype, d, E)) {
    nsplit = router_splits(n, d);
    float* dst = nsplit > 1 ? static_cast<float*>(ws) : logits;
    dim3 grid((n + kRouterRows - 1) / kRouterRows, nsplit, (E + kRouterCols - 1) / kRouterCols);
    hipLaunchKernelGGL(router_gemm_bf16_kernel, grid, dim3(256), 0, stream,
                       static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(Wg), n, d, E,
                       d / nsplit, dst);
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
  return launch_router_finalize(partial, nsplit, n, E, offset, score, logits, scores, scores_t,
                                stream);
}

hipError_t launch_router_finalize(const float* partial, int nsplit, int n, int E, const float* offset,
                                  int score, float* logits, float* scores, float* scores_t,
                                  hipStream_t stream) {
  const size_t lds = scores_t ? (size_t)kFinRows * (E + 1) * sizeof(float) : 0;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_finalize_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(router_finalize_kernel, dim3((n + kFinRows - 1) / kFinRows), dim3(1024), lds, stream, partial,
                     nsplit, n, E, offset, score, logits, scores, scores_t);
  return hipGetLastError();
}

}  // namespace moe
