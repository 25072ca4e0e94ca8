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
// 64 at a time through LDS tiles (rows padded by 16 bytes to spread banks);
// the next K tile is fetched from HBM into registers while the matrix cores
// work on the current one.  Two builds of the kernel: double-buffered LDS
// with two workgroups per CU, or one LDS copy with three (see the launcher).
//
// Scheduling: the per-expert tile counts are prefix-summed on the device
// (no host synchronisation), and a persistent grid walks the resulting tile
// list.  Workgroup b runs on XCD b % 8 (round-robin dispatch); each XCD takes
// a contiguous eighth of the tile list, with the N tiles of one M tile
// adjacent, so the workgroups that share an A panel (and a weight slice
// across neighbouring M tiles) share that XCD's L2.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
constexpr int kBM = 128;
constexpr int kBK = MOE_GEMM_BK;             // K per stage
constexpr int kLdsStride = kBK + 8;          // bf16 per LDS row
constexpr int kTileElems = 128 * kLdsStride; // one 128-row operand tile

constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;
#ifndef MOE_GEMM_ORDER
#define MOE_GEMM_ORDER -1                        // tile order: -1 by shape, 0 N inner, 1 M inner
#endif

enum { kEpiNone = 0, kEpiGelu = 1, kEpiSwiglu = 2 };

// GELU x * Phi(x) with erf from Abramowitz & Stegun formula 7.1.26
// (|error| <= 1.5e-7 over the real line, far below the bf16 rounding of the
// result): erf(z) = 1 - (a1 t + ... + a5 t^5) exp(-z^2), t = 1 / (1 + p z),
// z >= 0, odd extension for z < 0.
MOE_DEV float gelu_f(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __frcp_rn(1.0f + 0.3275911f * z);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float erf_z = 1.0f - poly * __expf(-z * z);
  const float erf_x = x < 0.f ? -erf_z : erf_z;
  return 0.5f * x * (1.0f + erf_x);
}
MOE_DEV float silu_f(float x) { return x * __frcp_rn(1.0f + __expf(-x)); }

// Tile list, built by every workgroup in LDS at kernel start (no separate
// launch, no host synchronisation): tile_off[e] = sum over e' < e of
// ceil(m_e' / kBM), tile_off[E] = all M tiles.  E <= kMaxExperts.
MOE_DEV void block_tile_plan(const int32_t* __restrict__ expert_offset, int E, int32_t* tile_off) {
  __shared__ int scratch[kGemmThreads / 64];
  constexpr int kPer = (kMaxExperts + kGemmThreads - 1) / kGemmThreads;
  const int e0 = threadIdx.x * kPer;
  int cnt[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = e0 + i;
    const int m = e < E ? expert_offset[e + 1] - expert_offset[e] : 0;
    cnt[i] = (m + kBM - 1) / kBM;
    sum += cnt[i];
  }
  int total = 0;
  int run = block_exclusive_scan<kGemmThreads>(sum, scratch, &total);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (e0 + i < E) tile_off[e0 + i] = run;
    run += cnt[i];
  }
  if (threadIdx.x == 0) tile_off[E] = total;
  __syncthreads();
}

template <bool kDual>
MOE_DEV int b_row_of(int r, int n0, int N) {
  // LDS B row r -> weight row.  Dual: rows 0..63 gate, 64..127 up (N is a
  // multiple of 64, so a dual tile is always full).  Single: a half tile at
  // the end of N re-reads the last row; those columns are never stored.
  if (!kDual) return min(n0 + r, N - 1);
  return r < 64 ? n0 + r : N + n0 + (r - 64);
}

// kLdsBufs = 2: double-buffered LDS stages (74 KB), two workgroups per CU.
// kLdsBufs = 1: one LDS copy (37 KB) and a register budget for three
// workgroups per CU; the stage in registers lands once every wave has left
// the LDS copy (one extra barrier per stage).
template <bool kDual, int kEpi, int kLdsBufs>
__global__ __launch_bounds__(kGemmThreads, kLdsBufs == 1 ? 3 : 1) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
    const int32_t* __restrict__ expert_offset, int E, int N, int K, int mt_inner,
    bf16_t* __restrict__ C) {
  // LDS: A and B K-stages, double buffered; reused for the output tile.
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * kLdsBufs * kTileElems];
  __shared__ int32_t tile_off[kMaxExperts + 1];
  block_tile_plan(expert_offset, E, tile_off);
  constexpr int kBNout = kDual ? 64 : 128;
  constexpr int kLoads = kBK / 16;                 // 16-byte loads per thread per operand and stage
  constexpr int kChunksRow = kBK / 8;              // 16-byte chunks per operand row
  constexpr int kRowsPass = kGemmThreads / kChunksRow;
  constexpr int kCStride = kBNout + 8;             // bf16 per output-tile row in LDS
  static_assert(128 * kCStride <= 2 * kLdsBufs * kTileElems, "output tile must fit the LDS stages");

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
  const int ld_row = tid / kChunksRow;
  const int ld_chunk = (tid % kChunksRow) * 8;
  const int nk = K / kBK;

  // Per-tile state: output placement and the global sources of this
  // thread's 16-byte staging loads.
  int row_base = 0, m_valid = 0, n0 = 0;
  const bf16_t* a_src[kLoads];
  const bf16_t* b_src[kLoads];
  auto setup = [&](int64_t t) {
    // expert owning tile t: expert e holds tiles [tile_off[e] * ntn, tile_off[e+1] * ntn)
    int e_lo = 0, e_hi = E - 1;
    while (e_lo < e_hi) {
      const int mid = (e_lo + e_hi + 1) >> 1;
      if ((int64_t)tile_off[mid] * ntn <= t) e_lo = mid; else e_hi = mid - 1;
    }
    const int e = e_lo;
    const int mtiles = tile_off[e + 1] - tile_off[e];
    const int local = (int)(t - (int64_t)tile_off[e] * ntn);
    // weight-streaming shapes walk an expert's M tiles innermost (its weight
    // slice is fetched once and the other M tiles hit L2); shapes with many
    // rows per expert walk N innermost (the A panel stays in L2)
    const int mloc = mt_inner ? local % mtiles : local / ntn;
    const int nt = mt_inner ? local / mtiles : local % ntn;
    row_base = expert_offset[e] + mloc * kBM;
    m_valid = min(kBM, expert_offset[e + 1] - row_base);
    n0 = nt * kBNout;
    const bf16_t* Be = B + (size_t)e * nbrows * K;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = ld_row + kRowsPass * i;
      a_src[i] = A + (size_t)(row_base + min(r, m_valid - 1)) * K + ld_chunk;   // tail rows re-read
      b_src[i] = Be + (size_t)b_row_of<kDual>(r, n0, N) * K + ld_chunk;
    }
  };
  u32x4_t ra[kLoads], rb[kLoads];
  auto load_stage = [&](int st) {
    const int koff = st * kBK;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + koff);
      rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + koff);
    }
  };
  auto store_stage = [&](int buf) {
    bf16_t* sA = smem + buf * kTileElems;
    bf16_t* sB = smem + (kLdsBufs + buf) * kTileElems;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      *reinterpret_cast<u32x4_t*>(&sA[(ld_row + kRowsPass * i) * kLdsStride + ld_chunk]) = ra[i];
      *reinterpret_cast<u32x4_t*>(&sB[(ld_row + kRowsPass * i) * kLdsStride + ld_chunk]) = rb[i];
    }
  };

  int64_t t = lo + blockIdx.x / kXcds;
  if (t >= hi) return;
  setup(t);
  load_stage(0);
  while (true) {
    // K pipeline: LDS double buffer; the next stage's global loads are in
    // flight while the matrix cores work on the current one.
    store_stage(0);
    if (nk > 1) load_stage(1);
    __syncthreads();
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kLdsBufs == 2 ? (kt & 1) : 0;
      const bf16_t* pa = smem + cur * kTileElems;
      const bf16_t* pb = smem + (kLdsBufs + cur) * kTileElems;
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
      if (kLdsBufs == 2) {
        if (kt + 1 < nk) {
          store_stage(cur ^ 1);
          if (kt + 2 < nk) load_stage(kt + 2);
        }
        __syncthreads();
      } else {
        // one LDS copy: every wave leaves it before the next stage lands
        __syncthreads();
        if (kt + 1 < nk) {
          store_stage(0);
          if (kt + 2 < nk) load_stage(kt + 2);
          __syncthreads();
        }
      }
    }

    // The next tile's first K stage starts loading before this tile's
    // epilogue, so HBM stays busy across the tile boundary.
    const int c_row_base = row_base, c_m_valid = m_valid, c_n0 = n0;
    const int64_t tn = t + per_xcd_blocks;
    if (tn < hi) {
      setup(tn);
      load_stage(0);
    }

    // Epilogue: activation, bf16 rounding, then the tile goes through LDS
    // so that global stores are whole 16-byte chunks of output rows.  The
    // stores are non-temporal: the output is read by the next kernel, not by
    // this one, and streaming it past the cache keeps the weight stream's
    // reads and these writes from contending for L2.
    // 32x32 accumulator layout: lane holds column (lane % 32), element v ->
    // row (v / 4) * 8 + (lane / 32) * 4 + v % 4.
    bf16_t* sC = smem;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + i * 32 + (v >> 2) * 8 + ((lane >> 5) << 2) + (v & 3);
        if (kDual) {
          const float g = acc[i][0][v], u = acc[i][1][v];
          sC[r * kCStride + wn * 32 + (lane & 31)] = f32_to_bf16(silu_f(g) * u);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float x = acc[i][j][v];
            if (kEpi == kEpiGelu) x = gelu_f(x);
            sC[r * kCStride + wn * 64 + j * 32 + (lane & 31)] = f32_to_bf16(x);
          }
        }
      }
    }
    __syncthreads();
    constexpr int kOutChunksRow = kBNout / 8;
    for (int q = tid; q < 128 * kOutChunksRow; q += kGemmThreads) {
      const int r = q / kOutChunksRow, c = (q % kOutChunksRow) * 8;
      if (r < c_m_valid && c_n0 + c < N)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sC + r * kCStride + c),
                                    reinterpret_cast<u32x4_t*>(C + (size_t)(c_row_base + r) * N + c_n0 + c));
    }
    __syncthreads();
    if (tn >= hi) break;
    t = tn;
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
  return align256((size_t)M_max * f * elem);
}

// Persistent grid: as many workgroups as fit on the device at once (so every
// one of them is resident and walks its share of the tile list), rounded
// down to a multiple of the XCD count.
template <typename Kern>
static int persistent_blocks(Kern kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                   kGemmThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  return ((per_cu * cus) / kXcds) * kXcds;
}

hipError_t launch_expert_ffn(const void* X_perm, int dtype, const int32_t* expert_offset, int E,
                             int d, int f, int act, const void* W1, const void* W2, int64_t M_max,
                             void* Y_perm, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  void* H = w;
  if (dtype == 1) {
    const bf16_t* x = static_cast<const bf16_t*>(X_perm);
    bf16_t* h = static_cast<bf16_t*>(H);
    // few rows per expert: the GEMMs stream weights, walk M tiles innermost
#if MOE_GEMM_ORDER < 0
    const int mt_inner = M_max <= (int64_t)E * 4 * kBM ? 1 : 0;
#else
    const int mt_inner = MOE_GEMM_ORDER;
#endif
    // Weight-streaming shapes (few rows per expert, M tiles innermost)
    // measured best with two double-buffered workgroups per CU; shapes with
    // many rows per expert (matrix-core bound) with three single-buffered
    // ones (2-3% faster there, 8-12% slower on weight streaming).
    const bool two_bufs = mt_inner != 0;
    auto gemm = [&](auto dual, auto epi, const bf16_t* a, const bf16_t* b, int N, int K, bf16_t* c) {
      constexpr bool kD = decltype(dual)::value;
      constexpr int kE = decltype(epi)::value;
      if (two_bufs) {
        static const int blocks = persistent_blocks(grouped_gemm_bf16_kernel<kD, kE, 2>);
        hipLaunchKernelGGL((grouped_gemm_bf16_kernel<kD, kE, 2>), dim3(blocks), dim3(kGemmThreads), 0, stream,
                           a, b, expert_offset, E, N, K, mt_inner, c);
      } else {
        static const int blocks = persistent_blocks(grouped_gemm_bf16_kernel<kD, kE, 1>);
        hipLaunchKernelGGL((grouped_gemm_bf16_kernel<kD, kE, 1>), dim3(blocks), dim3(kGemmThreads), 0, stream,
                           a, b, expert_offset, E, N, K, mt_inner, c);
      }
    };
    using std::integral_constant;
    if (act == 1)
      gemm(integral_constant<bool, true>{}, integral_constant<int, kEpiSwiglu>{}, x,
           static_cast<const bf16_t*>(W1), f, d, h);
    else
      gemm(integral_constant<bool, false>{}, integral_constant<int, kEpiGelu>{}, x,
           static_cast<const bf16_t*>(W1), f, d, h);
    gemm(integral_constant<bool, false>{}, integral_constant<int, kEpiNone>{}, h,
         static_cast<const bf16_t*>(W2), d, f, static_cast<bf16_t*>(Y_perm));
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
