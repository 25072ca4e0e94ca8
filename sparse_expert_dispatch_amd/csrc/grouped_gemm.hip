// Expert FFNs as a grouped GEMM over the expert-major buffer.
//
// MoE-routing pages: page 2 "Expert choice routing", section "The math"
// (Y[e] = Expert_e(X_in[e]) on dense per-expert batches, "ideal for batched
// matmuls") and section "A worked example" (the dense [E, k, d] batch);
// page 1 "Token choice vs expert choice routing", section "Dropped tokens
// flow in opposite directions" (dropless token choice moves the imbalance
// into kernel efficiency: ragged per-expert row counts).
//
// Per expert e with m_e rows (expert_offset, on the device):
//   up:   H = act(X_e W1_e^T)        GELU, or SwiGLU silu(X Wg^T) * (X Wu^T)
//   down: Y = H W2_e^T
// Both are "NT" products with K-contiguous operands, which is exactly what
// the MFMA operand layout wants: every lane feeds 8 consecutive K values of
// one row (A) or one column (B).
//
// bf16 kernel: a workgroup (4 waves) owns a 128-row x 128-column output
// tile (SwiGLU: 128 x 64 outputs from 64 gate + 64 up weight rows, so the
// gate and up accumulators of one output land in the same lane).  Each wave
// computes 64 x 64 with 2 x 2 v_mfma_f32_32x32x16_bf16 tiles.  K advances
// 64 at a time through double-buffered LDS tiles (rows padded by 16 bytes to
// spread banks); the next K tile is fetched from HBM into registers while
// the matrix cores work on the current one.
//
// Scheduling: the per-expert tile counts are prefix-summed on the device
// (no host synchronisation), and a persistent grid walks the resulting tile
// list.  Workgroup b runs on XCD b % 8 (round-robin dispatch); each XCD takes
// a contiguous eighth of the tile list, with the N tiles of one M tile
// adjacent, so the workgroups that share an A panel (and a weight slice
// across neighbouring M tiles) share that XCD's L2.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;
constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;          // bf16 per LDS row
constexpr int kTileElems = 128 * kLdsStride; // one 128-row operand tile
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;

enum { kEpiNone = 0, kEpiGelu = 1, kEpiSwiglu = 2 };

MOE_DEV float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
MOE_DEV float silu_f(float x) { return x / (1.0f + expf(-x)); }

// Tile list: tile_off[e] = sum over e' < e of ceil(m_e' / kBM).
__global__ __launch_bounds__(1024) void tile_plan_kernel(const int32_t* __restrict__ expert_offset,
                                                         int E, int32_t* __restrict__ tile_off) {
  __shared__ int scratch[16];
  const int e = threadIdx.x;
  int v = 0;
  for (int base = 0; base < E; base += 1024) {
    // E <= 1024 in practice; the loop keeps the kernel correct beyond that
    const int ee = base + e;
    const int m = ee < E ? expert_offset[ee + 1] - expert_offset[ee] : 0;
    const int tiles = (m + kBM - 1) / kBM;
    int total = 0;
    const int ex = block_exclusive_scan<1024>(tiles, scratch, &total);
    if (ee < E) tile_off[ee] = v + ex;
    v += total;
  }
  if (e == 0) tile_off[E] = v;
}

template <bool kDual>
MOE_DEV int b_row_of(int r, int n0, int N) {
  // LDS B row r -> weight row.  Dual: rows 0..63 gate, 64..127 up (N is a
  // multiple of 64, so a dual tile is always full).  Single: a half tile at
  // the end of N re-reads the last row; those columns are never stored.
  if (!kDual) return min(n0 + r, N - 1);
  return r < 64 ? n0 + r : N + n0 + (r - 64);
}

template <bool kDual, int kEpi>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ tile_off, int E, int N,
    int K, bf16_t* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][kTileElems];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][kTileElems];
  constexpr int kBNout = kDual ? 64 : 128;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + kBNout - 1) / kBNout;
  const int64_t n_tiles = (int64_t)tile_off[E] * ntn;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd_blocks = gridDim.x / kXcds;
  const int64_t lo = n_tiles * xcd / kXcds, hi = n_tiles * (xcd + 1) / kXcds;
  const int64_t nbrows = kDual ? 2 * (int64_t)N : (int64_t)N;

  // global->LDS copy assignment: thread covers rows (tid / 8) + 32 i, 16-byte chunk tid % 8
  const int ld_row = tid >> 3;
  const int ld_chunk = (tid & 7) << 3;

  for (int64_t t = lo + blockIdx.x / kXcds; t < hi; t += per_xcd_blocks) {
    const int mt = (int)(t / ntn);
    const int nt = (int)(t - (int64_t)mt * ntn);
    // expert owning M tile mt: last e with tile_off[e] <= mt
    int e_lo = 0, e_hi = E - 1;
    while (e_lo < e_hi) {
      const int mid = (e_lo + e_hi + 1) >> 1;
      if (tile_off[mid] <= mt) e_lo = mid; else e_hi = mid - 1;
    }
    const int e = e_lo;
    const int row_base = expert_offset[e] + (mt - tile_off[e]) * kBM;
    const int m_valid = min(kBM, expert_offset[e + 1] - row_base);
    const int n0 = nt * kBNout;
    const bf16_t* Be = B + (size_t)e * nbrows * K;

    const bf16_t* a_src[4];
    const bf16_t* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_row + 32 * i;
      const int ra = row_base + min(r, m_valid - 1);      // tail rows re-read the last valid row
      a_src[i] = A + (size_t)ra * K + ld_chunk;
      b_src[i] = Be + (size_t)b_row_of<kDual>(r, n0, N) * K + ld_chunk;
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    u32x4_t ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i]);
      rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4_t*>(&sA[0][(ld_row + 32 * i) * kLdsStride + ld_chunk]) = ra[i];
      *reinterpret_cast<u32x4_t*>(&sB[0][(ld_row + 32 * i) * kLdsStride + ld_chunk]) = rb[i];
    }
    __syncthreads();

    const int nk = K / kBK;
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        const int koff = (kt + 1) * kBK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + koff);
          rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + koff);
        }
      }
      const bf16_t* pa = sA[cur];
      const bf16_t* pb = sB[cur];
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        const int kc = s * 16 + ((lane >> 5) << 3);
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(pa + (wm * 64 + i * 32 + (lane & 31)) * kLdsStride + kc);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int brow = kDual ? (j * 64 + wn * 32 + (lane & 31)) : (wn * 64 + j * 32 + (lane & 31));
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(pb + brow * kLdsStride + kc);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (more) {
        const int nxt = cur ^ 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<u32x4_t*>(&sA[nxt][(ld_row + 32 * i) * kLdsStride + ld_chunk]) = ra[i];
          *reinterpret_cast<u32x4_t*>(&sB[nxt][(ld_row + 32 * i) * kLdsStride + ld_chunk]) = rb[i];
        }
      }
      __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane holds column (lane % 32),
    // element v -> row (v / 4) * 8 + (lane / 32) * 4 + v % 4.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + i * 32 + (v >> 2) * 8 + ((lane >> 5) << 2) + (v & 3);
        if (r >= m_valid) continue;
        bf16_t* crow = C + (size_t)(row_base + r) * N + n0;
        if (kDual) {
          const float g = acc[i][0][v], u = acc[i][1][v];
          crow[wn * 32 + (lane & 31)] = f32_to_bf16(silu_f(g) * u);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = wn * 64 + j * 32 + (lane & 31);
            if (n0 + col >= N) continue;
            float x = acc[i][j][v];
            if (kEpi == kEpiGelu) x = gelu_f(x);
            crow[col] = f32_to_bf16(x);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 path
// Plain fp32 FMA kernels (small fp32 layers): one thread per output.

MOE_DEV int expert_of_row(const int32_t* __restrict__ off, int E, int row) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_up_f32_kernel(const float* __restrict__ X,
                                                         const int32_t* __restrict__ off, int E, int d,
                                                         int f, int act, const float* __restrict__ W1,
                                                         float* __restrict__ H) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t M = off[E];
  if (i >= M * f) return;
  const int row = (int)(i / f), col = (int)(i - (int64_t)row * f);
  const int e = expert_of_row(off, E, row);
  const float* x = X + (size_t)row * d;
  const int rows = act == 1 ? 2 * f : f;
  const float* wg = W1 + ((size_t)e * rows + col) * d;
  float g = 0.f;
  for (int kk = 0; kk < d; ++kk) g = fmaf(x[kk], wg[kk], g);
  if (act == 1) {
    const float* wu = W1 + ((size_t)e * rows + f + col) * d;
    float u = 0.f;
    for (int kk = 0; kk < d; ++kk) u = fmaf(x[kk], wu[kk], u);
    H[i] = silu_f(g) * u;
  } else {
    H[i] = gelu_f(g);
  }
}

__global__ __launch_bounds__(256) void ffn_down_f32_kernel(const float* __restrict__ H,
                                                           const int32_t* __restrict__ off, int E,
                                                           int d, int f, const float* __restrict__ W2,
                                                           float* __restrict__ Y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t M = off[E];
  if (i >= M * d) return;
  const int row = (int)(i / d), col = (int)(i - (int64_t)row * d);
  const int e = expert_of_row(off, E, row);
  const float* h = H + (size_t)row * f;
  const float* w = W2 + ((size_t)e * d + col) * f;
  float y = 0.f;
  for (int kk = 0; kk < f; ++kk) y = fmaf(h[kk], w[kk], y);
  Y[i] = y;
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ffn_workspace_bytes(int64_t M_max, int E, int d, int f, int act, int dtype) {
  (void)d;
  (void)act;
  const size_t elem = dtype == 1 ? 2 : 4;
  return align256((size_t)(E + 1) * sizeof(int32_t)) + align256((size_t)M_max * f * elem);
}

static int persistent_blocks() {
  static int blocks = 0;
  if (!blocks) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    blocks = ((2 * cus + kXcds - 1) / kXcds) * kXcds;   // two workgroups per CU, multiple of 8
  }
  return blocks;
}

hipError_t launch_expert_ffn(const void* X_perm, int dtype, const int32_t* expert_offset, int E,
                             int d, int f, int act, const void* W1, const void* W2, int64_t M_max,
                             void* Y_perm, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  int32_t* tile_off = reinterpret_cast<int32_t*>(w);
  void* H = w + align256((size_t)(E + 1) * sizeof(int32_t));
  if (dtype == 1) {
    hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(1024), 0, stream, expert_offset, E, tile_off);
    const int blocks = persistent_blocks();
    const bf16_t* x = static_cast<const bf16_t*>(X_perm);
    bf16_t* h = static_cast<bf16_t*>(H);
    if (act == 1)
      hipLaunchKernelGGL((grouped_gemm_bf16_kernel<true, kEpiSwiglu>), dim3(blocks), dim3(kGemmThreads),
                         0, stream, x, static_cast<const bf16_t*>(W1), expert_offset, tile_off, E, f, d, h);
    else
      hipLaunchKernelGGL((grouped_gemm_bf16_kernel<false, kEpiGelu>), dim3(blocks), dim3(kGemmThreads),
                         0, stream, x, static_cast<const bf16_t*>(W1), expert_offset, tile_off, E, f, d, h);
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<false, kEpiNone>), dim3(blocks), dim3(kGemmThreads), 0,
                       stream, h, static_cast<const bf16_t*>(W2), expert_offset, tile_off, E, d, f,
                       static_cast<bf16_t*>(Y_perm));
  } else {
    const int64_t up = M_max * f, down = M_max * d;
    hipLaunchKernelGGL(ffn_up_f32_kernel, dim3((unsigned)((up + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(X_perm), expert_offset, E, d, f, act,
                       static_cast<const float*>(W1), static_cast<float*>(H));
    hipLaunchKernelGGL(ffn_down_f32_kernel, dim3((unsigned)((down + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(H), expert_offset, E, d, f,
                       static_cast<const float*>(W2), static_cast<float*>(Y_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
