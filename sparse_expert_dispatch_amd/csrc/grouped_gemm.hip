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
// Two bf16 kernels, both on v_mfma_f32_32x32x16_bf16:
//  - grouped_gemm_bf16_kernel (LDS kernel): a workgroup (4 waves) owns a
//    128-row output tile, 128 or 256 columns wide (SwiGLU: half as many
//    outputs from as many gate + up weight rows, so the gate and up
//    accumulators of one output land in the same lane); each wave computes
//    64 x 64 or 64 x 128.  K advances 64 at a time through LDS tiles; the
//    next K tile is fetched from HBM into registers while the matrix cores
//    work on the current one.  Weights in the natural layout or packed.
//  - stream_gemm_bf16_kernel (weight streaming, packed weights only): the
//    weights bypass LDS and stream into registers several K stages ahead
//    (see the kernel).
// The launcher picks the streaming kernel for packed weights when every
// expert has few rows (the GEMMs are bound by the weight stream), the LDS
// kernel with 128 x 256 tiles when experts have many rows (matrix-core
// bound), and the LDS kernel for the natural layout.
//
// Scheduling: the per-expert tile counts are prefix-summed on the device
// (no host synchronisation), and a persistent grid walks the resulting tile
// list.  Workgroup b runs on XCD b % 8 (round-robin dispatch); each XCD takes
// a contiguous eighth of the tile list, with the N tiles of one M tile
// adjacent, so the workgroups that share an A panel (and a weight slice
// across neighbouring M tiles) share that XCD's L2.
#include <type_traits>
#include <utility>

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

constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;
#ifndef MOE_GEMM_ORDER
#define MOE_GEMM_ORDER -1                        // tile order: -1 by shape, 0 N inner, 1 M inner
#endif

enum { kEpiNone = 0, kEpiGelu = 1, kEpiSwiglu = 2 };

// GELU x * Phi(x) with erf from Abramowitz & Stegun formula 7.1.26
// (|error| <= 1.5e-7 over the real line, far below the bf16 rounding of the
// result): erf(z) = 1 - (a1 t + ... + a5 t^5) exp(-z^2), t = 1 / (1 + p z),
// z >= 0, odd extension for z < 0.  The activation runs on every hidden
// element in the GEMM epilogue, where its VALU work stalls the matrix
// cores, so it is written for instruction count: the polynomial and the
// final scaling as fused multiply-adds, exp(-z^2) as the hardware's
// v_exp_f32 on -z^2 log2(e), and the reciprocals here and in SiLU as
// v_rcp_f32 (1 ulp).  About 15 VALU instructions per element.
MOE_DEV float gelu_f(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  const float q = fmaf(fmaf(fmaf(fmaf(1.061405429f, t, -1.453152027f), t, 1.421413741f), t, -0.284496736f), t,
                       0.254829592f);
  const float e = __builtin_amdgcn_exp2f((z * z) * -1.44269504088896341f);
  const float erf_z = fmaf(-(q * t), e, 1.0f);
  const float hx = 0.5f * x;
  return fmaf(hx, copysignf(erf_z, x), hx);
}
MOE_DEV float silu_f(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

// Two bf16 roundings in one v_cvt_pk_bf16_f32 (round to nearest even, the
// same bits as f32_to_bf16 for finite inputs); lo in bits 0..15.
MOE_DEV uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// The epilogue value of one accumulator element: SwiGLU silu(gate) * up,
// GELU, or the plain product.
template <int kEpi>
MOE_DEV float epi_value(float g, float u) {
  if (kEpi == kEpiSwiglu) return silu_f(g) * u;
  if (kEpi == kEpiGelu) return gelu_f(g);
  return g;
}

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

// Weight row of B-tile row r for a tile of kBRows weight rows at output
// column n0.  Dual (SwiGLU): rows [0, G) gate, [G, 2G) up, G = kBRows / 2.
// Rows past N re-read the last row; their output columns are never stored.
template <bool kDual, int kBRows>
MOE_DEV int b_row_of(int r, int n0, int N) {
  if (!kDual) return min(n0 + r, N - 1);
  constexpr int G = kBRows / 2;
  return r < G ? min(n0 + r, N - 1) : N + min(n0 + r - G, N - 1);
}

// kNB: 32-column MFMA blocks per wave in N (2: 64 x 64 per wave, 128 x 128
// tile; 4: 64 x 128 per wave, 128 x 256 tile, which reads 25% fewer LDS bytes
// per MFMA and each A panel once per 256 weight rows).
// kLdsBufs = 2: double-buffered LDS stages; 1: one LDS copy, the stage in
// registers lands once every wave has left it (one extra barrier per stage),
// which halves the LDS footprint (kNB = 2: three workgroups per CU instead
// of two; kNB = 4: two instead of one).
// kPacked: B is in the packed operand order written by pack_weights_kernel
// (each K stage of 32 weight rows is one contiguous 4 KB block; LDS holds
// the blocks unpadded and every fragment read is 64 consecutive 16-byte
// chunks); otherwise B is the natural [rows, K] layout.
template <bool kDual, int kEpi, int kLdsBufs, int kNB, bool kPacked>
__global__ __launch_bounds__(kGemmThreads, kNB == 4 ? 2 : (kLdsBufs == 1 ? 3 : 1)) void
grouped_gemm_bf16_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ row_index, int n_a,
                         const bf16_t* __restrict__ B, const int32_t* __restrict__ expert_offset, int E,
                         int N, int K, int mt_inner, bf16_t* __restrict__ C) {
  constexpr int kBRows = 2 * kNB * 32;             // weight rows per tile
  constexpr int kBNout = kDual ? kBRows / 2 : kBRows;
  constexpr int kTileA = 128 * kLdsStride;
  constexpr int kTileB = kPacked ? kBRows * kBK : kBRows * kLdsStride;
  static_assert(!kPacked || kBK == 64, "a packed K stage is 4 row-block chunks of 16 K");
  constexpr int kStageElems = kTileA + kTileB;
  constexpr int kChunksRow = kBK / 8;              // 16-byte chunks per operand row
  constexpr int kRowsPass = kGemmThreads / kChunksRow;
  constexpr int kLoadsA = 128 / kRowsPass;         // 16-byte loads per thread per stage
  constexpr int kLoadsB = kBRows / kRowsPass;
  constexpr int kPassCols = kBNout < 128 ? kBNout : 128;   // output columns per epilogue pass
  constexpr int kPasses = kBNout / kPassCols;
  constexpr int kCStride = kPassCols + 8;          // bf16 per output row in LDS
  static_assert(128 * kCStride <= kLdsBufs * kStageElems, "an epilogue pass must fit the LDS stages");
  // LDS: the K stage(s); reused for the output tile.
  __shared__ __attribute__((aligned(16))) bf16_t smem[kLdsBufs * kStageElems];
  __shared__ int32_t tile_off[kMaxExperts + 1];
  block_tile_plan(expert_offset, E, tile_off);

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

  // LDS row of this wave's B block j (32 weight rows from lane row 0)
  auto b_block_row = [&](int j) {
    if (!kDual) return wn * kNB * 32 + j * 32;
    constexpr int G = kBRows / 2, half = kNB / 2;
    return j < half ? wn * (G / 2) + j * 32 : G + wn * (G / 2) + (j - half) * 32;
  };
  // packed: tile-local row block of this wave's B block j (SwiGLU blocks
  // alternate gate, up for consecutive 32-column output blocks)
  auto b_block_packed = [&](int j) {
    if (!kDual) return wn * kNB + j;
    constexpr int half = kNB / 2;
    return j < half ? 2 * (wn * half + j) : 2 * (wn * half + j - half) + 1;
  };

  // Placement of tile t: expert e holds tiles [tile_off[e] * ntn,
  // tile_off[e+1] * ntn).  Weight-streaming shapes walk an expert's M tiles
  // innermost (its weight slice is fetched once and the other M tiles hit
  // L2); shapes with many rows per expert walk N innermost (the A panel
  // stays in L2).
  struct Place {
    int row_base, m_valid, n0, e;
  };
  auto place = [&](int64_t t) {
    int e_lo = 0, e_hi = E - 1;
    while (e_lo < e_hi) {
      const int mid = (e_lo + e_hi + 1) >> 1;
      if ((int64_t)tile_off[mid] * ntn <= t) e_lo = mid; else e_hi = mid - 1;
    }
    Place p;
    p.e = __builtin_amdgcn_readfirstlane(e_lo);
    const int mtiles = tile_off[p.e + 1] - tile_off[p.e];
    const int local = (int)(t - (int64_t)tile_off[p.e] * ntn);
    const int mloc = mt_inner ? local % mtiles : local / ntn;
    const int nt = mt_inner ? local / mtiles : local % ntn;
    p.row_base = __builtin_amdgcn_readfirstlane(expert_offset[p.e] + mloc * kBM);
    p.m_valid = __builtin_amdgcn_readfirstlane(min(kBM, expert_offset[p.e + 1] - p.row_base));
    p.n0 = __builtin_amdgcn_readfirstlane(nt * kBNout);
    return p;
  };
  // A rows of this thread's staging loads for tile t: the tile's slots, or
  // with row_index the rows of A those slots gather (the dispatch fused into
  // the GEMM); tail rows repeat the last valid one.  The rows of the next
  // tile are fetched one tile ahead (parked in LDS, which is cheaper than
  // registers here), so a gathered index is never waited on.
  __shared__ int nx_row[kLoadsA][kGemmThreads];
  auto rows_of = [&](int64_t t) {
    const Place p = place(min(t, hi - 1));
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const int s = p.row_base + min(ld_row + kRowsPass * i, p.m_valid - 1);
      nx_row[i][tid] = row_index ? min(max(row_index[s], 0), n_a - 1) : s;
    }
  };

  // Per-tile state (wave-uniform: kept in scalar registers) and, for the
  // natural B layout, the global sources of this thread's B loads.  Packed B
  // addresses are formed per load from the uniform tile base.
  int row_base = 0, m_valid = 0, n0 = 0;
  int a_row[kLoadsA];
  const bf16_t* b_tile = B;
  const bf16_t* b_src[kPacked ? 1 : kLoadsB];
  auto setup = [&](int64_t t) {
    const Place p = place(t);
    const int e = p.e;
    row_base = p.row_base;
    m_valid = p.m_valid;
    n0 = p.n0;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) a_row[i] = nx_row[i][tid];
    rows_of(t + per_xcd_blocks);
    // packed: expert e's row blocks in the first K stage's slab; natural: its matrix
    b_tile = kPacked ? B + (size_t)e * (nbrows / 32) * 2048 : B + (size_t)e * nbrows * K;
    if (!kPacked) {
#pragma unroll
      for (int i = 0; i < kLoadsB; ++i) {
        const int r = ld_row + kRowsPass * i;
        b_src[i] = b_tile + (size_t)b_row_of<kDual, kBRows>(r, n0, N) * K + ld_chunk;
      }
    }
  };
  u32x4_t ra[kLoadsA], rb[kLoadsB];
  auto load_stage = [&](int st) {
    const int koff = st * kBK;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i)
      ra[i] = *reinterpret_cast<const u32x4_t*>(A + (size_t)a_row[i] * K + ld_chunk + koff);
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) {
      if (kPacked) {
        // load i fetches tile-local row block i (columns past N re-read the last block)
        const int last = N / 32 - 1;
        const int pb = kDual ? 2 * min(n0 / 32 + (i >> 1), last) + (i & 1) : min(n0 / 32 + i, last);
        rb[i] = *reinterpret_cast<const u32x4_t*>(b_tile + ((size_t)st * E * (nbrows / 32) + pb) * 2048 +
                                                  tid * 8);
      } else {
        rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + koff);
      }
    }
  };
  auto store_stage = [&](int buf) {
    bf16_t* sA = smem + buf * kStageElems;
    bf16_t* sB = sA + kTileA;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i)
      *reinterpret_cast<u32x4_t*>(&sA[(ld_row + kRowsPass * i) * kLdsStride + ld_chunk]) = ra[i];
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) {
      if (kPacked)
        *reinterpret_cast<u32x4_t*>(&sB[i * kBK * 32 + tid * 8]) = rb[i];
      else
        *reinterpret_cast<u32x4_t*>(&sB[(ld_row + kRowsPass * i) * kLdsStride + ld_chunk]) = rb[i];
    }
  };

  int64_t t = lo + blockIdx.x / kXcds;
  if (t >= hi) return;
  rows_of(t);
  setup(t);
  load_stage(0);
  while (true) {
    // K pipeline: the next stage's global loads are in flight while the
    // matrix cores work on the current one.
    store_stage(0);
    if (nk > 1) load_stage(1);
    __syncthreads();
    f32x16_t acc[2][kNB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kLdsBufs == 2 ? (kt & 1) : 0;
      const bf16_t* pa = smem + cur * kStageElems;
      const bf16_t* pb = pa + kTileA;
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        const int kc = s * 16 + ((lane >> 5) << 3);
        bf16x8_t af[2], bfr[kNB];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(pa + (wm * 64 + i * 32 + (lane & 31)) * kLdsStride + kc);
#pragma unroll
        for (int j = 0; j < kNB; ++j)
          bfr[j] = kPacked
                       ? *reinterpret_cast<const bf16x8_t*>(pb + (b_block_packed(j) * (kBK / 16) + s) * 512 + lane * 8)
                       : *reinterpret_cast<const bf16x8_t*>(pb + (b_block_row(j) + (lane & 31)) * kLdsStride + kc);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < kNB; ++j)
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
    // (kPassCols output columns per pass) so that global stores are whole
    // 16-byte chunks of output rows.  The stores are non-temporal: the
    // output is read by the next kernel, not by this one, and streaming it
    // past the cache keeps the weight stream's reads and these writes from
    // contending for L2.
    // 32x32 accumulator layout: lane holds column (lane % 32), element v ->
    // row (v / 4) * 8 + (lane / 32) * 4 + v % 4.
    bf16_t* sC = smem;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      if (p > 0) __syncthreads();                  // the previous pass has been read out
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; v += 2) {         // elements v, v + 1: rows r, r + 1 of one column
          const int r = wm * 64 + i * 32 + (v >> 2) * 8 + ((lane >> 5) << 2) + (v & 3);
          if (kDual) {
#pragma unroll
            for (int j = 0; j < kNB / 2; ++j) {
              const int col = wn * (kBNout / 2) + j * 32 + (lane & 31);
              const uint32_t h = bf16x2_rne(epi_value<kEpi>(acc[i][j][v], acc[i][j + kNB / 2][v]),
                                            epi_value<kEpi>(acc[i][j][v + 1], acc[i][j + kNB / 2][v + 1]));
              sC[r * kCStride + col] = (bf16_t)h;
              sC[(r + 1) * kCStride + col] = (bf16_t)(h >> 16);
            }
          } else {
#pragma unroll
            for (int j = 0; j < kNB; ++j) {
              const int col = wn * kNB * 32 + j * 32 + (lane & 31);
              if (col / kPassCols != p) continue;
              const uint32_t h = bf16x2_rne(epi_value<kEpi>(acc[i][j][v], 0.f), epi_value<kEpi>(acc[i][j][v + 1], 0.f));
              sC[r * kCStride + col - p * kPassCols] = (bf16_t)h;
              sC[(r + 1) * kCStride + col - p * kPassCols] = (bf16_t)(h >> 16);
            }
          }
        }
      }
      __syncthreads();
      constexpr int kOutChunksRow = kPassCols / 8;
      const int pc0 = c_n0 + p * kPassCols;
      for (int q = tid; q < 128 * kOutChunksRow; q += kGemmThreads) {
        const int r = q / kOutChunksRow, c = (q % kOutChunksRow) * 8;
        if (r < c_m_valid && pc0 + c < N)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sC + r * kCStride + c),
                                      reinterpret_cast<u32x4_t*>(C + (size_t)(c_row_base + r) * N + pc0 + c));
      }
    }
    __syncthreads();
    if (tn >= hi) break;
    t = tn;
  }
}


// ---------------------------------------------------------------- weight-streaming kernel
// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
MOE_DEV void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Shapes with few rows per expert do little arithmetic per weight byte and
// are bound by the weight stream.  The LDS kernel above stages both
// operands through LDS, and at one to two waves per SIMD its compute phase
// alone (LDS writes, fragment reads, barriers) takes about as long as the
// weight stream, so the two barely overlap.  This kernel keeps the packed
// weights out of LDS: each wave owns all 128 rows of the tile and its own
// two 32-row weight blocks, and loads those blocks from HBM straight into
// registers in MFMA operand order (one contiguous 1 KB chunk per load
// instruction), kDepth K stages ahead, continuing across tile boundaries so
// the stream never drains.  Only A (the activations, L2-resident) goes
// through LDS, double-buffered, with one barrier per stage.
//
// Tile: 128 rows x 256 output columns (wave w: columns 64w .. 64w+63), or
// SwiGLU 128 x 128 (wave w: the gate and up blocks of columns 32w ..).  M
// tiles of an expert are innermost, as in the LDS kernel's weight-streaming
// order.  K / 64 must be a multiple of kDepth (the register ring is indexed
// at compile time); the launcher checks.
template <bool kDual, int kEpi, int kDepth>
__global__ __launch_bounds__(kGemmThreads, 1) void
stream_gemm_bf16_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ row_index, int n_a,
                        const bf16_t* __restrict__ Bp, const int32_t* __restrict__ expert_offset, int E,
                        int N, int K, bf16_t* __restrict__ C) {
  static_assert(kBK == 64, "a stage is four 16-K operand chunks");
  constexpr int kNW = kDual ? 128 : 256;           // output columns per tile
  constexpr int kCStride = kNW + 8;                // bf16 per output row in LDS
  constexpr int kATile = 128 * kLdsStride;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2 * kATile];
  __shared__ __attribute__((aligned(16))) bf16_t sC[128 * kCStride];
  __shared__ int32_t tile_off[kMaxExperts + 1];
  block_tile_plan(expert_offset, E, tile_off);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntn = (N + kNW - 1) / kNW;
  const int64_t n_tiles = (int64_t)tile_off[E] * ntn;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd_blocks = gridDim.x / kXcds;
  const int64_t lo = n_tiles * xcd / kXcds, hi = n_tiles * (xcd + 1) / kXcds;
  const int64_t t0 = lo + blockIdx.x / kXcds;
  if (t0 >= hi) return;
  const int ntiles = (int)((hi - t0 + per_xcd_blocks - 1) / per_xcd_blocks);
  const int nk = K / kBK;
  const int P = kDual ? 2 * N / 32 : N / 32;       // weight row blocks per expert
  const int last_pb = N / 32 - 1;
  const size_t stage_stride = (size_t)E * P * 2048;  // packed elements per K stage, all experts
  const int ld_row = tid >> 3, ld_chunk = (tid & 7) * 8;

  // Placement of this workgroup's j-th tile (M tiles of an expert innermost).
  struct Place {
    int row_base, m_valid, n0, e;
  };
  auto locate = [&](int j) {
    const int64_t t = t0 + (int64_t)j * per_xcd_blocks;
    int e_lo = 0, e_hi = E - 1;
    while (e_lo < e_hi) {
      const int mid = (e_lo + e_hi + 1) >> 1;
      if ((int64_t)tile_off[mid] * ntn <= t) e_lo = mid; else e_hi = mid - 1;
    }
    Place p;
    p.e = __builtin_amdgcn_readfirstlane(e_lo);
    const int mtiles = tile_off[p.e + 1] - tile_off[p.e];
    const int local = (int)(t - (int64_t)tile_off[p.e] * ntn);
    p.row_base = __builtin_amdgcn_readfirstlane(expert_offset[p.e] + (local % mtiles) * kBM);
    p.m_valid = __builtin_amdgcn_readfirstlane(min(kBM, expert_offset[p.e + 1] - p.row_base));
    p.n0 = __builtin_amdgcn_readfirstlane((local / mtiles) * kNW);
    return p;
  };

  // A rows of this thread's staging loads for tile j: the tile's slots, or
  // with row_index the rows of A those slots gather (the dispatch fused into
  // the GEMM); tail rows repeat the last valid one.
  auto rows_of = [&](int j, int (&rows)[4]) {
    const Place p = locate(min(j, ntiles - 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = p.row_base + min(ld_row + 32 * i, p.m_valid - 1);
      rows[i] = row_index ? min(max(row_index[s], 0), n_a - 1) : s;
    }
  };

  // Load cursor: the stage the next issue() fetches.  Past the last tile it
  // re-reads the last stage (in bounds, never used), so every iteration
  // issues the same loads and the compiler's memory-counter waits stay exact.
  // The A rows of the next tile are fetched one tile ahead.
  int l_j = 0, l_kt = 0;
  int l_row[4], nx_row[4];
  const bf16_t* l_b0 = Bp;
  const bf16_t* l_b1 = Bp;
  auto load_tile = [&](int j) {
    const Place p = locate(min(j, ntiles - 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) l_row[i] = nx_row[i];
    rows_of(j + 1, nx_row);
    int pb0, pb1;
    if (kDual) {
      const int ob = min(p.n0 / 32 + wave, last_pb);
      pb0 = 2 * ob;
      pb1 = 2 * ob + 1;
    } else {
      pb0 = min(p.n0 / 32 + 2 * wave, last_pb);
      pb1 = min(p.n0 / 32 + 2 * wave + 1, last_pb);
    }
    l_b0 = Bp + ((size_t)p.e * P + pb0) * 2048 + lane * 8;
    l_b1 = Bp + ((size_t)p.e * P + pb1) * 2048 + lane * 8;
  };
  u32x4_t ra[kDepth][4], rb[kDepth][2][4];
  auto issue = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int kt = l_j < ntiles ? l_kt : nk - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[slot][i] = *reinterpret_cast<const u32x4_t*>(A + (size_t)l_row[i] * K + ld_chunk + kt * kBK);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      rb[slot][0][s] = *reinterpret_cast<const u32x4_t*>(l_b0 + kt * stage_stride + s * 512);
      rb[slot][1][s] = *reinterpret_cast<const u32x4_t*>(l_b1 + kt * stage_stride + s * 512);
    }
    if (++l_kt == nk) {
      l_kt = 0;
      ++l_j;
      load_tile(l_j);
    }
  };
  int buf = 0;
  auto store_a = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(&sA[buf * kATile + (ld_row + 32 * i) * kLdsStride + ld_chunk]) = ra[slot][i];
  };

  using std::integral_constant;
  rows_of(0, nx_row);
  load_tile(0);
  static_for<0, kDepth>([&](auto u) { issue(u); });
  store_a(integral_constant<int, 0>{});
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][b][v] = 0.f;
    for (int kt0 = 0; kt0 < nk; kt0 += kDepth) {
      static_for<0, kDepth>([&](auto uc) {
        // one K stage: MFMAs on this stage's A (LDS) and B (ring slot U),
        // the next stage's A into the other LDS buffer, the slot refilled
        // kDepth stages ahead
        constexpr int U = decltype(uc)::value;
        const bf16_t* pa = sA + buf * kATile;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kc = s * 16 + ((lane >> 5) << 3);
          bf16x8_t af[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t*>(pa + (i * 32 + (lane & 31)) * kLdsStride + kc);
          const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, rb[U][0][s]);
          const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, rb[U][1][s]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], b0, acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], b1, acc[i][1], 0, 0, 0);
          }
        }
        buf ^= 1;
        store_a(integral_constant<int, (U + 1) % kDepth>{});
        issue(integral_constant<int, U>{});
        __syncthreads();
      });
    }

    // Epilogue: activation, bf16 rounding, the tile through LDS, whole
    // 16-byte chunks of output rows with non-temporal stores.  The loads of
    // the next tile's first stages are already in flight.  32x32
    // accumulator layout: lane holds column (lane % 32), element v -> row
    // (v / 4) * 8 + (lane / 32) * 4 + v % 4.
    const Place p = locate(j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) {           // elements v, v + 1: rows r, r + 1 of one column
        const int r = i * 32 + (v >> 2) * 8 + ((lane >> 5) << 2) + (v & 3);
        if (kDual) {
          const int col = wave * 32 + (lane & 31);
          const uint32_t h = bf16x2_rne(epi_value<kEpi>(acc[i][0][v], acc[i][1][v]),
                                        epi_value<kEpi>(acc[i][0][v + 1], acc[i][1][v + 1]));
          sC[r * kCStride + col] = (bf16_t)h;
          sC[(r + 1) * kCStride + col] = (bf16_t)(h >> 16);
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int col = wave * 64 + b * 32 + (lane & 31);
            const uint32_t h = bf16x2_rne(epi_value<kEpi>(acc[i][b][v], 0.f), epi_value<kEpi>(acc[i][b][v + 1], 0.f));
            sC[r * kCStride + col] = (bf16_t)h;
            sC[(r + 1) * kCStride + col] = (bf16_t)(h >> 16);
          }
        }
      }
    }
    __syncthreads();
    constexpr int kOutChunksRow = kNW / 8;
    for (int q = tid; q < 128 * kOutChunksRow; q += kGemmThreads) {
      const int r = q / kOutChunksRow, c = (q % kOutChunksRow) * 8;
      if (r < p.m_valid && p.n0 + c < N)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sC + r * kCStride + c),
                                    reinterpret_cast<u32x4_t*>(C + (size_t)(p.row_base + r) * N + p.n0 + c));
    }
  }
}

// ---------------------------------------------------------------- weight packing
// Packed operand order of the expert weights W [E, R, K] (bf16,
// K-contiguous; R % 32 == 0, K % 64 == 0).  Row block p of an expert holds
// 32 weight rows: rows 32p .. 32p+31, or for a SwiGLU W1 (R = 2F, gate rows
// first) the gate rows 32q .. of output block q at p = 2q and the matching
// up rows F + 32q .. at p = 2q + 1.  A 1 KB chunk holds, at 16-byte slot
// l = 0..63, the 8 values W[e][row(p, l % 32)][k0 + 8 (l / 32) + 0..7]:
// exactly the B operand of one v_mfma_f32_32x32x16_bf16 (32 output
// columns, 16 K).  Chunks are ordered K stage (64 K) first, then expert,
// row block, and the stage's four 16-K steps:
//   element ((((kt * E + e) * R/32 + p) * 4 + s) * 64 + l) * 8 + j
//   holds W[e][row(p, l % 32)][64 kt + 16 s + 8 (l / 32) + j].
// So one K stage of a GEMM tile (consecutive row blocks of one expert) is
// one contiguous run, and the tiles in flight at the same time (the same
// stage of neighbouring tiles) sit next to each other in memory, which
// keeps HBM row-buffer locality across the chip.
//
// One thread per 16-byte chunk: the writes are fully coalesced, each read
// is one 16-byte piece of a row.
__global__ __launch_bounds__(256) void pack_weights_kernel(const bf16_t* __restrict__ W, int64_t chunks,
                                                           int E, int R, int K, int gate_up,
                                                           bf16_t* __restrict__ P) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int lane = (int)(c & 63);
  const int s = (int)((c >> 6) & 3);
  const int64_t blk = c >> 8;                      // (kt * E + e) * R/32 + p
  const int nb = R / 32;
  const int p = (int)(blk % nb);
  const int64_t ke = blk / nb;
  const int e = (int)(ke % E);
  const int kt = (int)(ke / E);
  const int row = gate_up ? ((p & 1) ? R / 2 : 0) + (p >> 1) * 32 + (lane & 31) : p * 32 + (lane & 31);
  const int k0 = kt * 64 + s * 16 + (lane >> 5) * 8;
  *reinterpret_cast<u32x4_t*>(P + c * 8) =
      *reinterpret_cast<const u32x4_t*>(W + ((int64_t)e * R + row) * (int64_t)K + k0);
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


#ifndef MOE_GEMM_NB_STREAM
#define MOE_GEMM_NB_STREAM 2     // N blocks per wave, weight-streaming shapes
#endif
#ifndef MOE_GEMM_NB_MFMA
#define MOE_GEMM_NB_MFMA 4       // N blocks per wave, shapes with many rows per expert
#endif

#ifndef MOE_STREAM_DEPTH
#define MOE_STREAM_DEPTH 2       // K stages of packed weights in flight per wave, weight streaming
#endif

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

// One launch of a persistent kernel; the grid size is computed once per
// kernel (its occupancy does not change).
template <auto kKernel, typename... Args>
static void launch_persistent(hipStream_t stream, Args... args) {
  static const int blocks = persistent_blocks(kKernel);
  hipLaunchKernelGGL(kKernel, dim3(blocks), dim3(kGemmThreads), 0, stream, args...);
}

hipError_t launch_pack_weights(const void* W, int E, int R, int K, int gate_up, void* P,
                               hipStream_t stream) {
  const int64_t chunks = (int64_t)E * R * K / 8;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(W), chunks, E, R, K, gate_up, static_cast<bf16_t*>(P));
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const void* X_perm, const int32_t* row_index, int n_x, int dtype,
                             const int32_t* expert_offset, int E, int d, int f, int act, const void* W1,
                             const void* W2, int64_t M_max, void* Y_perm, void* ws, bool packed,
                             hipStream_t stream) {
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
    // measured best with 128 x 128 tiles and two double-buffered workgroups
    // per CU; shapes with many rows per expert (matrix-core bound) with
    // 128 x 256 tiles (a quarter fewer LDS bytes per MFMA) and one LDS copy,
    // two workgroups per CU (8-10% faster there, slower on weight streaming).
    const bool two_bufs = mt_inner != 0;
    // a_index / n_a: rows of A gathered through an index (the up GEMM with a
    // fused dispatch) or nullptr (A's rows are the slots)
    auto gemm = [&](auto dual, auto epi, const bf16_t* a, const int32_t* a_index, int n_a, const bf16_t* b,
                    int N, int K, bf16_t* c) {
      constexpr bool kD = decltype(dual)::value;
      constexpr int kE = decltype(epi)::value;
      const int nk = K / kBK;
      if (packed && mt_inner && nk % MOE_STREAM_DEPTH == 0) {
        launch_persistent<stream_gemm_bf16_kernel<kD, kE, MOE_STREAM_DEPTH>>(stream, a, a_index, n_a, b,
                                                                              expert_offset, E, N, K, c);
      } else if (two_bufs) {
        if (packed)
          launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 2, MOE_GEMM_NB_STREAM, true>>(
              stream, a, a_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
        else
          launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 2, MOE_GEMM_NB_STREAM, false>>(
              stream, a, a_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
      } else {
        if (packed)
          launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 1, MOE_GEMM_NB_MFMA, true>>(
              stream, a, a_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
        else
          launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 1, MOE_GEMM_NB_MFMA, false>>(
              stream, a, a_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
      }
    };
    using std::integral_constant;
    const int n_h = (int)M_max;
    if (act == 1)
      gemm(integral_constant<bool, true>{}, integral_constant<int, kEpiSwiglu>{}, x, row_index, n_x,
           static_cast<const bf16_t*>(W1), f, d, h);
    else
      gemm(integral_constant<bool, false>{}, integral_constant<int, kEpiGelu>{}, x, row_index, n_x,
           static_cast<const bf16_t*>(W1), f, d, h);
    gemm(integral_constant<bool, false>{}, integral_constant<int, kEpiNone>{}, h, nullptr, n_h,
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
