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
// bf16 kernels, all on v_mfma_f32_32x32x16_bf16:
//  - grouped_gemm_bf16_kernel (LDS kernel): each wave computes 64 x 64 or
//    64 x 128 (SwiGLU: half as many outputs from as many gate + up weight
//    rows, so the gate and up accumulators of one output land in the same
//    lane); K advances 64 at a time through LDS tiles, the next K tile
//    fetched from HBM into registers while the matrix cores work on the
//    current one.  A workgroup of 4 waves owns a 128-row tile, 128 or 256
//    columns wide; with packed weights, experts averaging 2048 rows or more
//    and an A operand past 2 GiB, a workgroup of 8 waves owns a 256 x 256
//    tile.  Weights in the natural layout or packed.
//  - grouped_gemm_dma_kernel (packed weights, many rows per expert): the
//    same 128 x 256 tiles with both operands moved into LDS by the buffer
//    loads' LDS mode, 32-K stages three deep, every fragment of a stage
//    read ahead of its matrix work (see the kernel);
//  - stream_pair_gemm_bf16_kernel (weight streaming, packed weights): the
//    weights bypass LDS and stream into registers two K stages ahead, two
//    4-wave halves per workgroup (see the kernel);
//    stream_gemm_bf16_kernel, its 4-wave predecessor, serves A operands of
//    more than 2 GiB (the paired kernel addresses A through 32-bit offsets).
// The launcher picks weight streaming for packed weights when every expert
// has few rows (the GEMMs are bound by the weight stream), the LDS-DMA
// kernel when experts have many rows (matrix-core bound), and the LDS
// kernel for the natural layout.
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
#ifndef MOE_PAIR_TALL_MAX
#define MOE_PAIR_TALL_MAX 192    // experts of 129 .. this many rows on tall tiles, the others on wide tiles
#endif
constexpr int kBM = 128;
constexpr int kBK = MOE_GEMM_BK;             // K per stage
constexpr int kLdsStride = kBK + 8;          // bf16 per LDS row

constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;
#ifndef MOE_GEMM_ORDER
#define MOE_GEMM_ORDER -1                        // tile order: -1 by shape, 0 N inner, 1 M inner
#endif

// kEpiF32: no activation, fp32 output (C is float*; the backward's
// pre-activation recompute)
enum { kEpiNone = 0, kEpiGelu = 1, kEpiSwiglu = 2, kEpiF32 = 3 };

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
// ceil(m_e' / kRows), tile_off[E] = all M tiles.  E <= kMaxExperts.
template <int kThreads = kGemmThreads, int kRows = kBM>
MOE_DEV void block_tile_plan(const int32_t* __restrict__ expert_offset, int E, int32_t* tile_off) {
  __shared__ int scratch[kThreads / 64];
  constexpr int kPer = (kMaxExperts + kThreads - 1) / kThreads;
  const int e0 = threadIdx.x * kPer;
  int cnt[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = e0 + i;
    const int m = e < E ? expert_offset[e + 1] - expert_offset[e] : 0;
    cnt[i] = (m + kRows - 1) / kRows;
    sum += cnt[i];
  }
  int total = 0;
  int run = block_exclusive_scan<kThreads>(sum, scratch, &total);
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
// kWM: waves in M (2: 4 waves, 128-row tiles; 4: 8 waves, 256-row tiles,
// one workgroup per CU with two waves per SIMD, double-buffered LDS: the
// same 64 x 128 wave tiles, with a quarter fewer global and LDS-write bytes
// per MFMA than two 128-row workgroups and one barrier per K stage).
// kBKs: B is stored K-major, W [E, K, N] (the backward's dX = dA W1: K runs
// down W1's rows), natural layout only, not SwiGLU.  A stage of B is staged
// as [64 K rows][tile columns + 8] with each group of 8 K rows permuted
// (logical row 8 g + 4 h + q at 8 g + 2 q + h), and a fragment is two
// ds_read_b64_tr_b16: within each 16-lane group the lanes address 4 rows x
// 16 columns (lane 4 a + b: row a, columns 4 b ..) and the transpose hands
// lane c column c of those rows, i.e. four consecutive K; lanes 32 .. 63
// take the next 8 K and lanes 16 .. 31 / 48 .. 63 the next 16 columns,
// which is the 32x32x16 B operand.  The row stride (tile columns + 8) keeps
// the rows a fragment read touches 4 banks apart.
template <bool kDual, int kEpi, int kLdsBufs, int kNB, bool kPacked, int kWM = 2, bool kBKs = false>
__global__ __launch_bounds__(kWM * 128, kWM == 4 ? 1 : (kNB == 4 ? 2 : (kLdsBufs == 1 ? 3 : 1))) void
grouped_gemm_bf16_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ row_index, int n_a,
                         const bf16_t* __restrict__ B, const int32_t* __restrict__ expert_offset, int E,
                         int N, int K, int mt_inner, bf16_t* __restrict__ C) {
  constexpr int kT = kWM * 128;                    // threads
  constexpr int kTM = kWM * 64;                    // rows per tile
  constexpr int kBRows = 2 * kNB * 32;             // weight rows per tile
  constexpr int kBNout = kDual ? kBRows / 2 : kBRows;
  constexpr int kTileA = kTM * kLdsStride;
  constexpr int kLdB = kBRows + 8;                 // K-major B: bf16 per LDS K row
  constexpr int kTileB = kPacked ? kBRows * kBK : (kBKs ? kBK * kLdB : kBRows * kLdsStride);
  static_assert(!kPacked || kBK == 64, "a packed K stage is 4 row-block chunks of 16 K");
  static_assert(!kBKs || (!kPacked && !kDual && kBK == 64 && kWM == 2), "K-major B: natural, not SwiGLU");
  constexpr int kStageElems = kTileA + kTileB;
  constexpr int kChunksRow = kBK / 8;              // 16-byte chunks per operand row
  constexpr int kRowsPass = kT / kChunksRow;
  constexpr int kLoadsA = kTM / kRowsPass;         // 16-byte loads per thread per stage
  constexpr int kLoadsB = kBRows / kRowsPass;
  constexpr int kPassCols = kBNout < 128 ? kBNout : 128;   // output columns per epilogue pass
  constexpr int kPasses = kBNout / kPassCols;
  constexpr int kCStride = kPassCols + 8;          // bf16 per output row in LDS
  static_assert(kTM * kCStride <= kLdsBufs * kStageElems, "an epilogue pass must fit the LDS stages");
  static_assert(kWM == 2 || kPacked, "256-row tiles: packed weights");
  // LDS: the K stage(s); reused for the output tile.
  __shared__ __attribute__((aligned(16))) bf16_t smem[kLdsBufs * kStageElems];
  __shared__ int32_t tile_off[kMaxExperts + 1];
  block_tile_plan<kT, kTM>(expert_offset, E, tile_off);

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
    p.row_base = __builtin_amdgcn_readfirstlane(expert_offset[p.e] + mloc * kTM);
    p.m_valid = __builtin_amdgcn_readfirstlane(min(kTM, expert_offset[p.e + 1] - p.row_base));
    p.n0 = __builtin_amdgcn_readfirstlane(nt * kBNout);
    return p;
  };
  // A rows of this thread's staging loads for tile t: the tile's slots, or
  // with row_index the rows of A those slots gather (the dispatch fused into
  // the GEMM); tail rows repeat the last valid one.  The rows of the next
  // tile are fetched one tile ahead (parked in LDS, which is cheaper than
  // registers here), so a gathered index is never waited on.
  __shared__ int nx_row[kLoadsA][kT];
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
  const bf16_t* b_src[kPacked || kBKs ? 1 : kLoadsB];
  // K-major B: buffer loads from the expert's W with one 32-bit byte offset
  // per load (K row and column inside the stage); the stage goes into the
  // scalar offset
  uint32_t b_voff[kBKs ? kLoadsB : 1];
  __amdgpu_buffer_rsrc_t b_rsrc;
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
    if (kBKs) {
      // K row c / (kBRows / 8) of the stage, columns 8 (c % (kBRows / 8)) ..
      // (past N: the last 8 columns again, never stored)
      b_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(b_tile), (short)0,
                                                 (int)min((int64_t)K * N * 2, (int64_t)0x7FFFFFFF), 0x00020000);
#pragma unroll
      for (int i = 0; i < kLoadsB; ++i) {
        const int c = tid + kT * i;
        const int kr = c / (kBRows / 8), cc = (c % (kBRows / 8)) * 8;
        b_voff[i] = (uint32_t)(kr * N + min(n0 + cc, N - 8)) * 2u;
      }
    } else if (!kPacked) {
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
        // load i fetches tile-local row block i (with 512 threads, blocks
        // 2i and 2i + 1, one per 256 threads; columns past N re-read the
        // last block)
        const int last = N / 32 - 1;
        const int bi = kT == 256 ? i : i * (kT / 256) + (tid >> 8);
        const int pb = kDual ? 2 * min(n0 / 32 + (bi >> 1), last) + (bi & 1) : min(n0 / 32 + bi, last);
        rb[i] = *reinterpret_cast<const u32x4_t*>(b_tile + ((size_t)st * E * (nbrows / 32) + pb) * 2048 +
                                                  (tid & 255) * 8);
      } else if (kBKs) {
        rb[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_voff[i], koff * N * 2, 0));
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
      if (kPacked) {
        *reinterpret_cast<u32x4_t*>(&sB[i * kT * 8 + tid * 8]) = rb[i];
      } else if (kBKs) {
        const int c = tid + kT * i;
        const int kr = c / (kBRows / 8);
        const int pr = (kr & ~7) | ((kr & 3) << 1) | ((kr >> 2) & 1);
        *reinterpret_cast<u32x4_t*>(&sB[pr * kLdB + (c % (kBRows / 8)) * 8]) = rb[i];
      } else {
        *reinterpret_cast<u32x4_t*>(&sB[(ld_row + kRowsPass * i) * kLdsStride + ld_chunk]) = rb[i];
      }
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
        for (int j = 0; j < kNB; ++j) {
          if (kBKs) {
            const bf16_t* q = pb + (s * 16 + 8 * (lane >> 5) + 2 * ((lane >> 2) & 3)) * kLdB + b_block_row(j) +
                              16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            typedef short v4i16_t __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
            const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)q);
            const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(q + kLdB));
            bfr[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            bfr[j] = kPacked
                         ? *reinterpret_cast<const bf16x8_t*>(pb + (b_block_packed(j) * (kBK / 16) + s) * 512 + lane * 8)
                         : *reinterpret_cast<const bf16x8_t*>(pb + (b_block_row(j) + (lane & 31)) * kLdsStride + kc);
          }
        }
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
    if constexpr (kEpi == kEpiF32) {
      // fp32 through LDS, 64 columns per pass (row stride 72 floats: the
      // fragment writes of rows r and r + 4 land 32 banks apart), then
      // 16-byte pieces of output rows
      constexpr int kFC = 64, kFS = kFC + 8;
      static_assert(kTM * kFS * 4 <= kLdsBufs * kStageElems * 2, "an fp32 pass fits the LDS stages");
      float* sCf = reinterpret_cast<float*>(smem);
      float* Cf = reinterpret_cast<float*>(C);
#pragma unroll
      for (int p = 0; p < kBNout / kFC; ++p) {
        if (p > 0) __syncthreads();                // the previous pass has been read out
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          const int cb = wn * kNB * 32 + j * 32;   // this block's first tile column
          if (cb / kFC != p) continue;             // uniform
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int r = wm * 64 + i * 32 + (v >> 2) * 8 + ((lane >> 5) << 2) + (v & 3);
              sCf[r * kFS + cb - p * kFC + (lane & 31)] = acc[i][j][v];
            }
        }
        __syncthreads();
        const int pc0 = c_n0 + p * kFC;
        for (int q = tid; q < kTM * (kFC / 4); q += kT) {
          const int r = q / (kFC / 4), c = (q % (kFC / 4)) * 4;
          if (r < c_m_valid && pc0 + c < N)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sCf + r * kFS + c),
                                        reinterpret_cast<u32x4_t*>(Cf + (size_t)(c_row_base + r) * N + pc0 + c));
        }
      }
    } else {
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
      for (int q = tid; q < kTM * kOutChunksRow; q += kT) {
        const int r = q / kOutChunksRow, c = (q % kOutChunksRow) * 8;
        if (r < c_m_valid && pc0 + c < N)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sC + r * kCStride + c),
                                      reinterpret_cast<u32x4_t*>(C + (size_t)(c_row_base + r) * N + pc0 + c));
      }
    }
    }
    __syncthreads();
    if (tn >= hi) break;
    t = tn;
  }
}


// ---------------------------------------------------------------- LDS-DMA kernel
// The matrix-core-bound shapes (many rows per expert, packed weights) on
// 128 x 256 tiles of 4 waves, two workgroups per CU, with the operands
// moved from memory straight into LDS by the buffer loads' LDS mode (each
// 16-byte lane load lands at the wave's LDS base + 16 x lane) instead of
// through registers.  That frees the 48 registers the staged kernel keeps
// for the next K tile, and both K steps' fragments of a stage are read
// before its matrix work.  Stages are 32 K deep; three LDS stages rotate: at
// the top of stage g (after its barrier) the loads of stage g + 2 are
// issued into the buffer that stage g - 1 used, so two stages are always in
// flight, and a tile's first stages are fetched during the previous tile's
// last stages and epilogue (a load cursor that runs across tiles, as in the
// weight-streaming kernel).
//   A: 128 rows x 64 bytes per stage; row r, 16-byte chunk c is stored at
//      slot c ^ swz(r), swz(r) = ((r >> 1) ^ (r >> 3)) & 3, so that the 32
//      rows a fragment read touches at one K chunk fall on distinct banks
//      (the loads pick their source chunk to match).
//   B: the packed operand order's 1 KB chunks (32 weight rows x 16 K), in
//      the staged kernel's tile-local block order.
// Waits are explicit: the LDS-mode loads are assembly the compiler does
// not see, so nothing but the kernel's own waits orders the LDS reads after
// them.  Each stage waits until at most the next stage's six loads per wave
// are outstanding (vmcnt counts in issue order; the epilogue's stores and
// the compiler's own loads only make that wait stricter), then a barrier
// publishes the stage; compiler-only memory clobbers keep the LDS reads on
// their side of the barrier.
constexpr int kDmaBK = 32;
constexpr int kDmaBufs = 3;
constexpr int kDmaStageA = kBM * kDmaBK * 2;        // bytes
constexpr int kDmaStageB = 256 * kDmaBK * 2;
constexpr int kDmaStage = kDmaStageA + kDmaStageB;  // 24 KB
constexpr int kDmaPerWave = 6;                      // LDS-mode loads per wave and stage (2 A, 4 B)

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_t;

// Buffer resource for 32-bit offsets from base (raw, no swizzle).
MOE_DEV i32x4_t dma_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (i32x4_t){(int32_t)(uint32_t)a, (int32_t)((uint32_t)(a >> 32) & 0xFFFFu), (int32_t)num_records,
                   0x00020000};
}
// One LDS-mode buffer load: every lane's 16 bytes at rsrc + soff + voff land
// at LDS byte lds + 16 x lane.  Written as assembly so that the compiler
// neither sees an LDS write (it would otherwise wait for every such load
// before any LDS read) nor counts the load: the kernel waits for it with
// explicit s_waitcnt.  No register output (nothing the compiler could take
// as written early); M0 is set in the same block, with the one wait state
// an LDS-mode load needs after an M0 write (the kernels that use it keep
// nothing else in M0).
MOE_DEV void dma16(i32x4_t rsrc, uint32_t voff, int32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
               : "m0");
}
// The same with 4 bytes per lane (LDS byte lds + 4 x lane).
MOE_DEV void dma4(i32x4_t rsrc, uint32_t voff, int32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
               : "m0");
}
MOE_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_char_t*)p);
}

MOE_DEV int dma_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// s_waitcnt with vmcnt(n) (n < 64) and lgkmcnt(0), expcnt left alone
template <int n>
MOE_DEV void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}
MOE_DEV void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool kDual, int kEpi>
__global__ __launch_bounds__(kGemmThreads, 2) void
grouped_gemm_dma_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ row_index, int n_a,
                        const bf16_t* __restrict__ B, const int32_t* __restrict__ expert_offset, int E, int N,
                        int K, int mt_inner, bf16_t* __restrict__ C) {
  constexpr int kT = kGemmThreads, kTM = kBM, kNB = 4, kBRows = 256;
  constexpr int kBNout = kDual ? kBRows / 2 : kBRows;
  constexpr int kPassCols = 64, kCStride = kPassCols + 8;
  static_assert(kTM * kCStride * 2 <= kDmaStage, "an epilogue pass fits one LDS stage");
  __shared__ __attribute__((aligned(1024))) char smem[kDmaBufs * kDmaStage];
  __shared__ int32_t tile_off[kMaxExperts + 1];
  block_tile_plan<kT, kTM>(expert_offset, E, tile_off);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + kBNout - 1) / kBNout;
  const int64_t n_tiles = (int64_t)__builtin_amdgcn_readfirstlane(tile_off[E]) * ntn;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd_blocks = gridDim.x / kXcds;
  const int64_t lo = n_tiles * xcd / kXcds, hi = n_tiles * (xcd + 1) / kXcds;
  const int P = kDual ? 2 * N / 32 : N / 32;      // packed row blocks per expert
  const int last_pb = N / 32 - 1;
  const int nk = K / kDmaBK;

  // packed tile-local row block of this wave's B block j (as the staged kernel)
  auto b_block_packed = [&](int j) __attribute__((always_inline)) {
    if (!kDual) return wn * kNB + j;
    constexpr int half = kNB / 2;
    return j < half ? 2 * (wn * half + j) : 2 * (wn * half + j - half) + 1;
  };
  struct Place {
    int row_base, m_valid, n0, e;
  };
  auto place = [&](int64_t t) __attribute__((always_inline)) {
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
    p.row_base = __builtin_amdgcn_readfirstlane(expert_offset[p.e] + mloc * kTM);
    p.m_valid = __builtin_amdgcn_readfirstlane(min(kTM, expert_offset[p.e + 1] - p.row_base));
    p.n0 = __builtin_amdgcn_readfirstlane(nt * kBNout);
    return p;
  };
  // The gathered A rows of the cursor's tile j sit in s_idx[j & 1]: the
  // index entries of a tile's 128 rows, loaded in LDS mode by waves 0 and 1
  // when the cursor enters the tile before it (at least two stages, hence
  // two waits and barriers, before they are read; the slot refilled was
  // last read at least one barrier earlier), so no index load is ever
  // waited on at once.  The first two tiles' entries are loaded up front.
  __shared__ __attribute__((aligned(16))) int32_t s_idx[2][kTM];
  const i32x4_t idx_rsrc = dma_rsrc(row_index, (uint32_t)__builtin_amdgcn_readfirstlane(expert_offset[E]) * 4u);
  const i32x4_t a_rsrc = dma_rsrc(A, (uint32_t)min((int64_t)n_a * K * 2, (int64_t)0x7FFFFFFF));
  const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t idx_base = __builtin_amdgcn_readfirstlane(lds_addr(&s_idx[0][0]));
  auto fetch_idx = [&](int64_t tt, int slot) __attribute__((always_inline)) {
    if (row_index && wave < 2) {
      const Place p = place(min(tt, hi - 1));
      dma4(idx_rsrc, (uint32_t)(p.row_base + wave * 64 + lane) * 4u, 0, idx_base + slot * kTM * 4 + wave * 256);
    }
  };
  // Load cursor: tile d_t (the d_j-th of this workgroup), stage d_kt.  Past
  // the workgroup's last tile it stays on that tile's last stage and
  // re-reads it, so every stage issues the same loads.
  int64_t d_t = lo + blockIdx.x / kXcds;
  if (d_t >= hi) return;
  int d_kt = 0, d_e = 0, d_n0 = 0, d_j = 0;
  uint32_t a_voff[2];
  auto cursor_tile = [&](int fetch) __attribute__((always_inline)) {
    const Place p = place(d_t);
    d_e = p.e;
    d_n0 = p.n0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * (4 * i + wave) + (lane >> 2);
      const int c = (lane & 3) ^ dma_swz(r);
      const int rr = min(r, p.m_valid - 1);
      const int row = row_index ? min(max(s_idx[d_j & 1][rr], 0), n_a - 1) : p.row_base + rr;
      a_voff[i] = (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)(c * 16);
    }
    if (fetch) fetch_idx(d_t + per_xcd_blocks, (d_j + 1) & 1);
    ++d_j;
  };
  auto issue = [&](int dbuf) __attribute__((always_inline)) {
    const int kt = __builtin_amdgcn_readfirstlane(d_kt);
    const int de = __builtin_amdgcn_readfirstlane(d_e), dn0 = __builtin_amdgcn_readfirstlane(d_n0);
    const uint32_t base = smem_base + dbuf * kDmaStage;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(a_rsrc, a_voff[i], kt * kDmaBK * 2, base + (4 * i + wave) * 1024);
    // packed B: 64-K stage kt / 2 of expert d_e, chunks 2 (kt & 1) + s
    const i32x4_t b_rsrc = dma_rsrc(B + ((size_t)(kt >> 1) * E + de) * P * 2048, 0x7FFFFFFF);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 4 * i + wave, bi = q >> 1, s = q & 1;
      const int pb = kDual ? 2 * min(dn0 / 32 + (bi >> 1), last_pb) + (bi & 1) : min(dn0 / 32 + bi, last_pb);
      dma16(b_rsrc, (uint32_t)lane * 16, pb * 4096 + ((kt & 1) * 2 + s) * 1024, base + kDmaStageA + q * 1024);
    }
    if (d_kt + 1 < nk) {
      ++d_kt;
    } else if (d_t + per_xcd_blocks < hi) {
      d_kt = 0;
      d_t += per_xcd_blocks;
      cursor_tile(1);
    }
  };

  fetch_idx(d_t, 0);
  fetch_idx(d_t + per_xcd_blocks, 1);
  wait_vm_lgkm0<0>();
  lds_barrier();
  cursor_tile(0);
  int64_t t = d_t;                                 // the first tile computed (the cursor may pass it below)
  int cbuf = 0;
  issue(0);
  lds_barrier();                                   // s_idx[0] read by every wave before it is refilled
  issue(1);
  const int sw = dma_swz(lane & 31);
  while (true) {
    const Place pc = place(t);
    f32x16_t acc[2][kNB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      // this stage's loads done (the next stage's may still be in flight),
      // every wave's reads of the buffer about to be refilled done
      wait_vm_lgkm0<kDmaPerWave>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(cbuf == 0 ? 2 : cbuf - 1);
      const char* pa = smem + cbuf * kDmaStage;
      const char* pb = pa + kDmaStageA;
      bf16x8_t af[2][2], bfr[2][kNB];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = (2 * s + (lane >> 5)) ^ sw;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[s][i] = *reinterpret_cast<const bf16x8_t*>(pa + (wm * 64 + i * 32 + (lane & 31)) * 64 + c * 16);
#pragma unroll
        for (int j = 0; j < kNB; ++j)
          bfr[s][j] = *reinterpret_cast<const bf16x8_t*>(pb + (b_block_packed(j) * 2 + s) * 1024 + lane * 16);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < kNB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s][i], bfr[s][j], acc[i][j], 0, 0, 0);
      cbuf = cbuf == 2 ? 0 : cbuf + 1;
    }

    // Epilogue in the last stage's buffer (the next tile's first two stages
    // are landing in the other two): activation, bf16 rounding, 64 output
    // columns per pass through LDS, whole 16-byte chunks of output rows
    // stored non-temporally.  32x32 accumulator layout: lane holds column
    // (lane % 32), element v -> row (v / 4) * 8 + (lane / 32) * 4 + v % 4.
    bf16_t* sC = reinterpret_cast<bf16_t*>(smem + (cbuf == 0 ? 2 : cbuf - 1) * kDmaStage);
    if (!kDual && kEpi != kEpiNone) {
      // the activation in place, one 32 x 32 block at a time
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = epi_value<kEpi>(acc[i][j][v], 0.f);
        }
    }
    constexpr int kEpiPack = kDual ? kEpi : kEpiNone;
#pragma unroll
    for (int p = 0; p < kBNout / kPassCols; ++p) {
      lds_barrier();                               // the stage (or the previous pass) has been read
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_barrier(0);         // one row block's activations at a time
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int r = wm * 64 + i * 32 + (v >> 2) * 8 + ((lane >> 5) << 2) + (v & 3);
          if (kDual) {
            if (wn != p) continue;                 // uniform: a wave's 64 outputs are one pass
#pragma unroll
            for (int j = 0; j < kNB / 2; ++j) {
              const int col = j * 32 + (lane & 31);
              const uint32_t h = bf16x2_rne(epi_value<kEpi>(acc[i][j][v], acc[i][j + kNB / 2][v]),
                                            epi_value<kEpi>(acc[i][j][v + 1], acc[i][j + kNB / 2][v + 1]));
              sC[r * kCStride + col] = (bf16_t)h;
              sC[(r + 1) * kCStride + col] = (bf16_t)(h >> 16);
            }
          } else {
#pragma unroll
            for (int j = 0; j < kNB; ++j) {
              if (wn * 2 + (j >> 1) != p) continue;  // uniform
              const int col = (j & 1) * 32 + (lane & 31);
              const uint32_t h = bf16x2_rne(epi_value<kEpiPack>(acc[i][j][v], 0.f),
                                            epi_value<kEpiPack>(acc[i][j][v + 1], 0.f));
              sC[r * kCStride + col] = (bf16_t)h;
              sC[(r + 1) * kCStride + col] = (bf16_t)(h >> 16);
            }
          }
        }
      }
      lds_barrier();
      const int pc0 = pc.n0 + p * kPassCols;
#pragma unroll
      for (int q = tid; q < kTM * (kPassCols / 8); q += kT) {
        const int r = q / (kPassCols / 8), c = (q % (kPassCols / 8)) * 8;
        if (r < pc.m_valid && pc0 + c < N)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sC + r * kCStride + c),
                                      reinterpret_cast<u32x4_t*>(C + (size_t)(pc.row_base + r) * N + pc0 + c));
      }
    }
    if (t + per_xcd_blocks >= hi) break;
    t += per_xcd_blocks;
  }
  // the cursor's re-reads of the last stage are still landing
  __builtin_amdgcn_s_waitcnt(0x0070 | 0xF00);     // vmcnt(0)
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

// ---------------------------------------------------------------- paired weight-streaming kernel
// Weight streaming with two 4-wave halves per workgroup (8 waves, two per
// SIMD), so that no weight byte is fetched twice and each SIMD has a second
// wave to issue matrix work while the first waits on memory.  A tile is
// chosen per expert from its row count m:
//  - wide: 128 rows x 2 kNW output columns; half h takes the columns
//    n0 + h kNW ..: twice the distinct weight bytes in flight per CU.  An
//    expert of more rows takes ceil(m / 128) row tiles per column block,
//    adjacent in the list, so neighbouring workgroups of one XCD stream the
//    same weights at about the same time and the re-reads meet in the cache;
//  - tall (128 < m <= MOE_PAIR_TALL_MAX): 256 rows x kNW columns; half h
//    takes rows 128 h .. of the same columns, so both halves load the same
//    weight chunks at the same K stage (the second load is served by the
//    cache) and the expert streams its weights once, from one CU.  This
//    pays while the second half is sparse; an expert whose second 128 rows
//    are mostly full, or of more than 256 rows (two tall row tiles far
//    apart in the list), measured faster on wide row tiles (top-8-of-256
//    routing: up 3450 -> 3076 us, down 1790 -> 1699 us; Switch top-1 with
//    160-row experts unchanged).
// Each wave owns 128 rows and two 32-row weight blocks (64 output columns,
// or the gate and up blocks of 32 SwiGLU outputs) as in the 4-wave kernel;
// the weights stream from memory straight into registers, kDepth K stages
// ahead, and only A (the token rows) goes through LDS.  All global loads are
// buffer loads: the uniform part of an address is scalar and each lane keeps
// a 32-bit offset.
constexpr int kPairThreads = 512;

// Tile plan of the paired kernel, two lists in expert order: the wide tiles
// (ceil(m / 128) * ceil(N / (2 kNW)) per expert not on tall tiles, M tiles
// innermost; wide_off[e] = wide tiles of experts before e) and the tall
// tiles (ceil(m / 256) * ceil(N / kNW) per expert of 129 ..
// MOE_PAIR_TALL_MAX rows, M tiles innermost; tall_off[e]).  wide_off[E],
// tall_off[E] are the totals.
template <int kNW>
MOE_DEV void pair_tile_plan(const int32_t* __restrict__ expert_offset, int E, int N, int32_t* wide_off,
                            int32_t* tall_off) {
  __shared__ int scratch[kPairThreads / 64];
  static_assert(kMaxExperts <= kPairThreads, "one expert per thread");
  const int ntw = (N + 2 * kNW - 1) / (2 * kNW), ntn = (N + kNW - 1) / kNW;
  const int e = threadIdx.x;
  const int m = e < E ? expert_offset[e + 1] - expert_offset[e] : 0;
  const bool tall = m > 128 && m <= MOE_PAIR_TALL_MAX;
  const int cw = (m > 0 && !tall) ? ((m + 127) / 128) * ntw : 0;
  const int ct = tall ? ((m + 255) / 256) * ntn : 0;
  int tot_w = 0, tot_t = 0;
  const int rw = block_exclusive_scan<kPairThreads>(cw, scratch, &tot_w);
  const int rt = block_exclusive_scan<kPairThreads>(ct, scratch, &tot_t);
  if (e < E) {
    wide_off[e] = rw;
    tall_off[e] = rt;
  }
  if (threadIdx.x == 0) {
    wide_off[E] = tot_w;
    tall_off[E] = tot_t;
  }
  __syncthreads();
}

template <bool kDual, int kEpi, int kDepth>
__global__ __launch_bounds__(kPairThreads, 1) void
stream_pair_gemm_bf16_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ row_index, int n_a,
                             const bf16_t* __restrict__ Bp, const int32_t* __restrict__ expert_offset, int E,
                             int N, int K, bf16_t* __restrict__ C, int32_t* __restrict__ tile_ctr) {
  static_assert(kBK == 64, "a stage is four 16-K operand chunks");
  constexpr int kNW = kDual ? 128 : 256;           // output columns per half
  constexpr int kCStride = kNW + 8;                // bf16 per output row in LDS
  constexpr int kATile = 256 * kLdsStride;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2 * kATile];
  __shared__ __attribute__((aligned(16))) bf16_t sC[128 * kCStride];   // one half per pass
  __shared__ int32_t wide_off[kMaxExperts + 1], tall_off[kMaxExperts + 1];
  // A row offsets (bytes) of this thread's staging loads, one table per tile
  // parity; each thread reads and writes only its own entries
  __shared__ __attribute__((aligned(16))) uint32_t row_off[2][kPairThreads][4];
  pair_tile_plan<kNW>(expert_offset, E, N, wide_off, tall_off);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave >> 2, qw = wave & 3;         // half, wave within the half
  // Schedule: XCD x (workgroups b with b % 8 == x share its L2) takes an
  // eighth of the wide list and an eighth of the tall list, in that order.
  // Wide tiles carry twice the weight bytes of tall ones, and tall tiles
  // whose halves both hold rows twice the matrix work, so tiles differ in
  // cost and a static deal leaves some workgroups with far more work than
  // others.  Each workgroup therefore takes its first two tiles round-robin
  // (positions w and w + 32 of its XCD's sequence) and every further tile
  // from the XCD's counter tile_ctr[x] (zero at launch): whoever finishes
  // first takes the next tile.  Neighbouring workgroups of an XCD still work
  // on neighbouring tiles of the same expert (shared A rows, and for an
  // expert's M tiles shared weights, in that L2).
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd_blocks = gridDim.x / kXcds;
  const int n_wide = wide_off[E], n_tall = tall_off[E];
  const int wl = (int)((int64_t)n_wide * xcd / kXcds), wh = (int)((int64_t)n_wide * (xcd + 1) / kXcds);
  const int tl = (int)((int64_t)n_tall * xcd / kXcds), th = (int)((int64_t)n_tall * (xcd + 1) / kXcds);
  const int len = (wh - wl) + (th - tl);
  // Positions of this workgroup's tiles, three ahead of the one being
  // computed (the load pipeline locates tile j + 1 during tile j and gathers
  // the A rows of tile j + 2): slot j % 4 holds the j-th position; once the
  // sequence is exhausted a slot repeats the last valid position with
  // valid = 0.  Thread 0 writes a slot at the top of tile j - 3; the K loop's
  // barriers publish it long before it is read.
  __shared__ int tpos[4], tval[4];
  auto take = [&](int slot, int prev) {            // thread 0 only
    int p = len;
    if (tval[prev]) p = 2 * per_xcd_blocks + atomicAdd(&tile_ctr[xcd], 1);
    tpos[slot] = p < len ? p : tpos[prev];
    tval[slot] = p < len;
  };
  if (tid == 0) {
    const int w0 = blockIdx.x / kXcds;
    tpos[0] = w0;
    tval[0] = w0 < len;
    tval[1] = w0 + per_xcd_blocks < len;
    tpos[1] = tval[1] ? w0 + per_xcd_blocks : w0;
    take(2, 1);
  }
  __syncthreads();
  if (!tval[0]) return;
  auto valid = [&](int j) { return tval[j & 3] != 0; };
  const int nk = K / kBK;
  const int P = kDual ? 2 * N / 32 : N / 32;       // weight row blocks per expert
  const int last_pb = N / 32 - 1;
  const size_t stage_bytes = (size_t)E * P * 4096;  // packed bytes per K stage, all experts
  const int ld_row = tid >> 3, ld_chunk = (tid & 7) * 8;

  struct Place {
    int row_base, m_valid, n0, e, wide;
  };
  auto find = [&](const int32_t* off, int g) {     // expert holding list entry g
    int e_lo = 0, e_hi = E - 1;
    while (e_lo < e_hi) {
      const int mid = (e_lo + e_hi + 1) >> 1;
      if (off[mid] <= g) e_lo = mid; else e_hi = mid - 1;
    }
    return __builtin_amdgcn_readfirstlane(e_lo);
  };
  auto locate = [&](int j) {
    const int pos = tpos[j & 3];
    Place p;
    if (pos < wh - wl) {
      const int g = wl + pos;
      p.e = find(wide_off, g);
      p.wide = 1;
      const int base = expert_offset[p.e];
      const int m = expert_offset[p.e + 1] - base;
      const int mt = (m + 127) / 128;
      const int local = g - wide_off[p.e];
      p.row_base = __builtin_amdgcn_readfirstlane(base + (local % mt) * 128);
      p.m_valid = __builtin_amdgcn_readfirstlane(min(128, m - (local % mt) * 128));
      p.n0 = __builtin_amdgcn_readfirstlane((local / mt) * 2 * kNW);
    } else {
      const int g = tl + pos - (wh - wl);
      p.e = find(tall_off, g);
      const int base = expert_offset[p.e];
      const int m = expert_offset[p.e + 1] - base;
      const int mt = (m + 255) / 256;
      const int local = g - tall_off[p.e];
      p.wide = 0;
      p.row_base = __builtin_amdgcn_readfirstlane(base + (local % mt) * 256);
      p.m_valid = __builtin_amdgcn_readfirstlane(min(256, m - (local % mt) * 256));
      p.n0 = __builtin_amdgcn_readfirstlane((local / mt) * kNW);
    }
    return p;
  };

  // the A rows of tile j this thread stages (rows past the tile's last
  // repeat it; they feed only output rows that are never stored)
  auto rows_of = [&](int j) {
    const Place p = locate(j);
    uint32_t r4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = p.row_base + min(ld_row + 64 * i, p.m_valid - 1);
      const int r = row_index ? min(max(row_index[s], 0), n_a - 1) : s;
      r4[i] = (uint32_t)r * (uint32_t)(K * 2) + (uint32_t)(ld_chunk * 2);
    }
    *reinterpret_cast<u32x4_t*>(&row_off[j & 1][tid][0]) = (u32x4_t){r4[0], r4[1], r4[2], r4[3]};
  };

  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(A), (short)0, (int)min((int64_t)n_a * K * 2, (int64_t)0x7FFFFFFF), 0x00020000);
  const uint32_t b_lane = (uint32_t)lane * 16;

  // Load cursor (as in the 4-wave kernel): past the last tile it re-reads the
  // last stage of the last tile (locate() of an exhausted slot gives that
  // tile), so every iteration issues the same loads.
  int l_j = 0, l_kt = 0;
  const char* l_b = reinterpret_cast<const char*>(Bp);   // this wave's first row block, stage 0
  int l_b1 = 0;                                           // byte offset of its second row block
  auto load_tile = [&](int j) {
    const Place p = locate(j);
    rows_of(j + 1);
    const int nc = p.n0 + (p.wide ? hw * kNW : 0);        // this half's first output column
    int pb0, pb1;
    if (kDual) {
      const int ob = min(nc / 32 + qw, last_pb);
      pb0 = 2 * ob;
      pb1 = 2 * ob + 1;
    } else {
      pb0 = min(nc / 32 + 2 * qw, last_pb);
      pb1 = min(nc / 32 + 2 * qw + 1, last_pb);
    }
    l_b = reinterpret_cast<const char*>(Bp) + ((size_t)p.e * P + pb0) * 4096;
    l_b1 = __builtin_amdgcn_readfirstlane((pb1 - pb0) * 4096);
  };
  u32x4_t ra[kDepth][4], rb[kDepth][2][4];
  // The loads of the stage at the cursor come in two parts: issue_b(slot, s)
  // fetches the weight chunks of K step s, as soon as this stage's MFMAs of
  // step s have read that register pair, so the weight stream never waits
  // for the whole stage; issue_a then fetches the A rows and advances the
  // cursor.
  auto issue_b = [&](auto slot_c, auto step_c) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int s = decltype(step_c)::value;
    const int kt = valid(l_j) ? l_kt : nk - 1;
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(l_b + (size_t)kt * stage_bytes), (short)0, 0x7FFFFFFF, 0x00020000);
    rb[slot][0][s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_lane + s * 1024, 0, 0));
    rb[slot][1][s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_lane + s * 1024, l_b1, 0));
  };
  auto issue_a = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int kt = valid(l_j) ? l_kt : nk - 1;
    const u32x4_t ro = *reinterpret_cast<const u32x4_t*>(&row_off[l_j & 1][tid][0]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, ro[i], kt * 128, 0));
    if (++l_kt == nk) {
      l_kt = 0;
      ++l_j;
      load_tile(l_j);
    }
  };
  auto issue = [&](auto slot_c) {
    static_for<0, 4>([&](auto sc) { issue_b(slot_c, sc); });
    issue_a(slot_c);
  };
  int buf = 0;
  auto store_a = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(&sA[buf * kATile + (ld_row + 64 * i) * kLdsStride + ld_chunk]) = ra[slot][i];
  };

  using std::integral_constant;
  rows_of(0);
  load_tile(0);
  static_for<0, kDepth>([&](auto u) { issue(u); });
  store_a(integral_constant<int, 0>{});
  __syncthreads();

  for (int j = 0; valid(j); ++j) {
    if (tid == 0) take((j + 3) & 3, (j + 2) & 3);
    const Place pj = locate(j);
    const int r0 = pj.wide ? 0 : 128 * hw;         // this wave's first row in the tile
    // 32-row blocks of this wave holding rows of the expert (0..4, uniform
    // per wave): the matrix work follows the row count rounded up to 32
    const int nbw = min(4, max(0, (pj.m_valid - r0 + 31) >> 5));
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][b][v] = 0.f;
    for (int kt0 = 0; kt0 < nk; kt0 += kDepth) {
      static_for<0, kDepth>([&](auto uc) {
        constexpr int U = decltype(uc)::value;
        const bf16_t* pa = sA + buf * kATile + r0 * kLdsStride;
        // K step s of every row block, then step s's weight registers of
        // this ring slot are refilled for the stage kDepth ahead
        static_for<0, 4>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          const int kc = s * 16 + ((lane >> 5) << 3);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (i < nbw) {
              const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(pa + (i * 32 + (lane & 31)) * kLdsStride + kc);
              acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8_t, rb[U][0][s]),
                                                                  acc[i][0], 0, 0, 0);
              acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8_t, rb[U][1][s]),
                                                                  acc[i][1], 0, 0, 0);
            }
          }
          issue_b(integral_constant<int, U>{}, sc);
        });
        buf ^= 1;
        store_a(integral_constant<int, (U + 1) % kDepth>{});
        issue_a(integral_constant<int, U>{});
        __syncthreads();
      });
    }

    // Epilogue, one half per pass: the half's waves apply the activation,
    // round to bf16 and write their rows into LDS; then every thread stores
    // whole 16-byte chunks of output rows (non-temporal).  Wide tiles: pass
    // h covers columns n0 + h kNW ..; tall tiles: rows 128 h ...  32x32
    // accumulator layout: lane holds column (lane % 32), element v -> row
    // (v / 4) * 8 + (lane / 32) * 4 + v % 4.
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int prow = pj.wide ? 0 : 128 * ph;      // first tile row of this pass
      const int pcol = pj.n0 + (pj.wide ? ph * kNW : 0);
      const int m_pass = min(128, pj.m_valid - prow);
      if (m_pass <= 0 || pcol >= N) break;         // uniform
      if (ph > 0) __syncthreads();                 // the previous pass has been read out
      if (hw == ph) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int v = 0; v < 16; v += 2) {       // elements v, v + 1: rows r, r + 1 of one column
            const int r = i * 32 + (v >> 2) * 8 + ((lane >> 5) << 2) + (v & 3);
            if (kDual) {
              const int col = qw * 32 + (lane & 31);
              const uint32_t h = bf16x2_rne(epi_value<kEpi>(acc[i][0][v], acc[i][1][v]),
                                            epi_value<kEpi>(acc[i][0][v + 1], acc[i][1][v + 1]));
              sC[r * kCStride + col] = (bf16_t)h;
              sC[(r + 1) * kCStride + col] = (bf16_t)(h >> 16);
            } else {
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                const int col = qw * 64 + b * 32 + (lane & 31);
                const uint32_t h =
                    bf16x2_rne(epi_value<kEpi>(acc[i][b][v], 0.f), epi_value<kEpi>(acc[i][b][v + 1], 0.f));
                sC[r * kCStride + col] = (bf16_t)h;
                sC[(r + 1) * kCStride + col] = (bf16_t)(h >> 16);
              }
            }
          }
        }
      }
      __syncthreads();
      constexpr int kOutChunksRow = kNW / 8;
      for (int q = tid; q < 128 * kOutChunksRow; q += kPairThreads) {
        const int r = q / kOutChunksRow, c = (q % kOutChunksRow) * 8;
        if (r < m_pass && pcol + c < N)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(sC + r * kCStride + c),
                                      reinterpret_cast<u32x4_t*>(C + (size_t)(pj.row_base + prow + r) * N + pcol + c));
      }
    }
  }
}

// Clears the paired kernel's tile counters before a launch (a kernel rather
// than a memset, so that a captured graph replays it as it runs eagerly).
__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
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
#ifndef MOE_GEMM_WM_MFMA
#define MOE_GEMM_WM_MFMA 4       // waves in M there, packed weights (4: 256-row tiles, 8 waves)
#endif

#ifndef MOE_STREAM_DEPTH
#define MOE_STREAM_DEPTH 2       // K stages of packed weights in flight per wave, weight streaming
#endif
#ifndef MOE_GEMM_DMA
#define MOE_GEMM_DMA 1           // many rows per expert, packed: operands into LDS by the loads' LDS mode
#endif
#ifndef MOE_STREAM_PAIR
#define MOE_STREAM_PAIR 1        // weight streaming on the paired (8-wave) kernel
#endif

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ffn_workspace_bytes(int64_t M_max, int E, int d, int f, int act, int dtype) {
  (void)d;
  (void)act;
  const size_t elem = dtype == 1 ? 2 : 4;
  // H, then the grouped GEMMs' tile counters (bf16); nothing without rows
  if (M_max <= 0) return 0;
  return align256((size_t)M_max * f * elem) + (dtype == 1 ? kGemmWsBytes : 0);
}

// Persistent grid: as many workgroups as fit on the device at once (so every
// one of them is resident and walks its share of the tile list), rounded
// down to a multiple of the XCD count.
template <typename Kern>
static int persistent_blocks(Kern kernel, int threads = kGemmThreads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                   threads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  return ((per_cu * cus) / kXcds) * kXcds;
}

// One launch of a persistent kernel; the grid size is computed once per
// kernel (its occupancy does not change).
template <auto kKernel, int kThreads = kGemmThreads, typename... Args>
static void launch_persistent(hipStream_t stream, Args... args) {
  static const int blocks = persistent_blocks(kKernel, kThreads);
  hipLaunchKernelGGL(kKernel, dim3(blocks), dim3(kThreads), 0, stream, args...);
}

hipError_t launch_pack_weights(const void* W, int E, int R, int K, int gate_up, void* P,
                               hipStream_t stream) {
  const int64_t chunks = (int64_t)E * R * K / 8;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(W), chunks, E, R, K, gate_up, static_cast<bf16_t*>(P));
  return hipGetLastError();
}

// One grouped GEMM of the FFN on bf16: the up projection (stage 1: A = the
// token rows, through row_index when given; B = W1; activation epilogue; C =
// H [M_max, f]) or the down projection (stage 2: A = H; B = W2; C = Y_perm).
// ctr: kGemmWsBytes of device memory for the paired kernel's tile counters
// (cleared here before the launch).
static void launch_ffn_gemm_bf16(int stage, const bf16_t* a, const int32_t* row_index, int n_a,
                                 const int32_t* expert_offset, int E, int d, int f, int act, const bf16_t* b,
                                 int64_t M_max, bf16_t* c, bool packed, int32_t* ctr, hipStream_t stream) {
  // few rows per expert: the GEMMs stream weights, walk M tiles innermost.
  // The down projection on packed weights streams up to twice as many rows
  // per expert: its K (= f) is short, so the matrix-core kernel's per-tile
  // start and epilogue weigh more there (dropless top-8 of 64, 1024 rows
  // per expert on average: down 341 -> 317 us; the up projection measured
  // the same on either kernel and stays on the matrix-core one).
#if MOE_GEMM_ORDER < 0
  const int stream_rows = (packed && stage == 2) ? 8 * kBM : 4 * kBM;
  const int mt_inner = M_max <= (int64_t)E * stream_rows ? 1 : 0;
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
  auto gemm = [&](auto dual, auto epi, int N, int K) {
    constexpr bool kD = decltype(dual)::value;
    constexpr int kE = decltype(epi)::value;
    const int nk = K / kBK;
    if (packed && mt_inner && nk % MOE_STREAM_DEPTH == 0 && MOE_STREAM_PAIR &&
        (int64_t)n_a * K * 2 <= (int64_t)0x7FFFFFFF) {
      hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, stream, ctr, kXcds);
      launch_persistent<stream_pair_gemm_bf16_kernel<kD, kE, MOE_STREAM_DEPTH>, kPairThreads>(
          stream, a, row_index, n_a, b, expert_offset, E, N, K, c, ctr);
    } else if (packed && mt_inner && nk % MOE_STREAM_DEPTH == 0) {
      launch_persistent<stream_gemm_bf16_kernel<kD, kE, MOE_STREAM_DEPTH>>(stream, a, row_index, n_a, b,
                                                                            expert_offset, E, N, K, c);
    } else if (two_bufs) {
      if (packed)
        launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 2, MOE_GEMM_NB_STREAM, true>>(
            stream, a, row_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
      else
        launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 2, MOE_GEMM_NB_STREAM, false>>(
            stream, a, row_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
    } else {
      // Packed weights: the LDS-DMA kernel (A addressed through 32-bit
      // offsets); it measured 4-7% faster than the register-staged kernel on
      // the dropless top-8 projections and 5% faster than the 256 x 256
      // tiles on the always-on shared expert.  Past 2 GiB of A: 256-row
      // tiles once experts average 2048 rows or more (the shared expert's
      // shape: there the 8-wave tile measured 7% faster than 128-row
      // tiles; with fewer rows per expert its coarser tail per expert costs
      // more than that), else the staged 128 x 256 kernel.
      if (packed && MOE_GEMM_DMA && (int64_t)n_a * K * 2 <= (int64_t)0x7FFFFFFF)
        launch_persistent<grouped_gemm_dma_kernel<kD, kE>>(stream, a, row_index, n_a, b, expert_offset, E, N, K,
                                                           mt_inner, c);
      else if (packed && MOE_GEMM_WM_MFMA == 4 && M_max >= (int64_t)2048 * E)
        launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 2, MOE_GEMM_NB_MFMA, true, 4>, 512>(
            stream, a, row_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
      else if (packed)
        launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 1, MOE_GEMM_NB_MFMA, true>>(
            stream, a, row_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
      else
        launch_persistent<grouped_gemm_bf16_kernel<kD, kE, 1, MOE_GEMM_NB_MFMA, false>>(
            stream, a, row_index, n_a, b, expert_offset, E, N, K, mt_inner, c);
    }
  };
  using std::integral_constant;
  if (stage == 1) {
    if (act == 1)
      gemm(integral_constant<bool, true>{}, integral_constant<int, kEpiSwiglu>{}, f, d);
    else
      gemm(integral_constant<bool, false>{}, integral_constant<int, kEpiGelu>{}, f, d);
  } else {
    gemm(integral_constant<bool, false>{}, integral_constant<int, kEpiNone>{}, d, f);
  }
}

// The backward's pre-activation recompute C = A W^T per expert (rows
// grouped by expert_offset; A [rows, K], W [E, N, K] natural layout, both
// bf16; C [rows, N] fp32), on the LDS-tiled kernel with the same tile
// choice as the forward on natural weights.  K % 64 == 0.
hipError_t launch_rows_gemm_f32(const void* A, const int32_t* expert_offset, int E, const void* W, int N, int K,
                                int64_t M_max, float* C, hipStream_t stream) {
  const int mt_inner = M_max <= (int64_t)E * 4 * kBM ? 1 : 0;
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(W);
  bf16_t* c = reinterpret_cast<bf16_t*>(C);
  if (mt_inner)
    launch_persistent<grouped_gemm_bf16_kernel<false, kEpiF32, 2, MOE_GEMM_NB_STREAM, false>>(
        stream, a, nullptr, (int)M_max, b, expert_offset, E, N, K, mt_inner, c);
  else
    launch_persistent<grouped_gemm_bf16_kernel<false, kEpiF32, 1, MOE_GEMM_NB_MFMA, false>>(
        stream, a, nullptr, (int)M_max, b, expert_offset, E, N, K, mt_inner, c);
  return hipGetLastError();
}

// The backward's dX = dA W per expert with W stored K-major ([E, K, N]: the
// natural W1 read down its rows), bf16 out, on the LDS-tiled kernel.
// K % 64 == 0, N % 8 == 0.
hipError_t launch_rows_gemm_kmajor(const void* A, const int32_t* expert_offset, int E, const void* W, int N, int K,
                                   int64_t M_max, void* C, hipStream_t stream) {
  const int mt_inner = M_max <= (int64_t)E * 4 * kBM ? 1 : 0;
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(W);
  bf16_t* c = static_cast<bf16_t*>(C);
  if (mt_inner)
    launch_persistent<grouped_gemm_bf16_kernel<false, kEpiNone, 2, MOE_GEMM_NB_STREAM, false, 2, true>>(
        stream, a, nullptr, (int)M_max, b, expert_offset, E, N, K, mt_inner, c);
  else
    launch_persistent<grouped_gemm_bf16_kernel<false, kEpiNone, 1, MOE_GEMM_NB_MFMA, false, 2, true>>(
        stream, a, nullptr, (int)M_max, b, expert_offset, E, N, K, mt_inner, c);
  return hipGetLastError();
}

hipError_t launch_expert_gemm(int stage, const void* A, const int32_t* row_index, int n_a,
                              const int32_t* expert_offset, int E, int d, int f, int act, const void* W,
                              int64_t M_max, void* C, bool packed, void* ws, hipStream_t stream) {
  launch_ffn_gemm_bf16(stage, static_cast<const bf16_t*>(A), row_index, n_a, expert_offset, E, d, f, act,
                       static_cast<const bf16_t*>(W), M_max, static_cast<bf16_t*>(C), packed,
                       static_cast<int32_t*>(ws), stream);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const void* X_perm, const int32_t* row_index, int n_x, int dtype,
                             const int32_t* expert_offset, int E, int d, int f, int act, const void* W1,
                             const void* W2, int64_t M_max, void* Y_perm, void* ws, bool packed,
                             hipStream_t stream) {
  void* H = ws;
  if (dtype == 1) {
    int32_t* ctr = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align256((size_t)M_max * f * 2));
    launch_ffn_gemm_bf16(1, static_cast<const bf16_t*>(X_perm), row_index, n_x, expert_offset, E, d, f, act,
                         static_cast<const bf16_t*>(W1), M_max, static_cast<bf16_t*>(H), packed, ctr, stream);
    launch_ffn_gemm_bf16(2, static_cast<const bf16_t*>(H), nullptr, (int)M_max, expert_offset, E, d, f, act,
                         static_cast<const bf16_t*>(W2), M_max, static_cast<bf16_t*>(Y_perm), packed, ctr, stream);
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
