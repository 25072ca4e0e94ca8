// Router: Z = X W_g (+ per-expert offset), then the specified score
// transform (softmax over experts, or a sigmoid per expert).
//
// MoE-routing pages: page 2 "Expert choice routing", section "The math"
// (S = softmax(X W_g), X: [n, d], W_g: [d, E]); page 5 "MoE routing
// strategies explained", strategy 4 (sigmoid scores).
//
// bf16 with at most 64 experts: one fused kernel (GEMM on the matrix cores
// with W_g read in its [d, E] layout through LDS transpose reads, K split
// over the waves of a workgroup and summed in wave order, then offset,
// noise, scores and their transpose), no intermediate in memory.  bf16 with
// more experts: a split-K GEMM kernel (128-row x 64-expert tiles, each K
// stage of W_g transposed on its way into LDS; K split across workgroups,
// up to 8 slices, until the grid fills the GPU) writes per-slice partial
// logits to the workspace, and a finalize kernel adds the slices in slice
// order (deterministic), adds the offset and evaluates the scores.  fp32,
// or shapes the matrix-core tiling does not cover: a scalar GEMM, then the
// finalize kernel.

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

// Scores of one row held as lane l, register j -> expert l + 64 j (entries
// with j >= nj or l + 64 j >= E are ignored): the softmax over the row
// (score 0: max, exp of the differences, halving-tree sum, quotient) or
// the per-expert sigmoid / sqrtsoftplus.  Both router paths call it, so
// they produce the same bits from the same logits.
template <int R>
MOE_DEV void row_scores(const float (&z)[R], int nj, int E, int score, float (&p)[R]) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  if (score == 0) {
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < nj && lane + 64 * j < E) m = fmaxf(m, z[j]);
    m = wave_max_f32(m);
    float t[R];
#pragma unroll
    for (int j = 0; j < R; ++j) t[j] = (j < nj && lane + 64 * j < E) ? spec_exp(z[j] - m) : 0.f;
    const float s = row_tree_sum(t, next_pow2(E));
#pragma unroll
    for (int j = 0; j < R; ++j) p[j] = t[j] / s;
  } else {
#pragma unroll
    for (int j = 0; j < R; ++j) p[j] = spec_expert_score(z[j], score);
  }
}

// Fused router for up to 64 experts: the GEMM, the offset and noise, the
// scores and their transpose in one kernel, with no K-split partials in
// memory.  A workgroup owns 16 RT token rows and all E experts; its KW
// waves split K (wave w takes the w-th d / KW slice) and each keeps 16 RT x
// E accumulators (v_mfma_f32_16x16x32_bf16).  Per 32-wide K step a wave
// copies the 32 x 64 block of W_g [d, E] as loaded (row-major, no
// transpose) into its own LDS rows, and reads the matrix-core B fragments
// back with ds_read_b64_tr_b16: within each 16-lane group, lane 4q + e
// receives element e of the 4-element runs addressed by lanes q, q + 4,
// q + 8, q + 12.  Pointing lane i of a group at row (i / 4) and experts
// 4 (i % 4) .. +3 of the block therefore hands lane r four consecutive K
// values of expert r; two such reads make the 8-value fragment.  The waves'
// LDS regions are private, so the K loop has no barrier.  The partial
// accumulators are then added through LDS in wave order (deterministic),
// and the rows finish as in the finalize kernel.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

#ifndef MOE_ROUTER_AHEAD
#define MOE_ROUTER_AHEAD 4
#endif
#ifndef MOE_ROUTER_KW_BIG
#define MOE_ROUTER_KW_BIG 8
#endif
#ifndef MOE_ROUTER_KW_SMALL
#define MOE_ROUTER_KW_SMALL 16
#endif
constexpr int kFusedAhead = MOE_ROUTER_AHEAD;   // K steps in flight per wave

// LDS of the fused kernel with NT 16-expert tiles per workgroup (expert
// tile of 16 NT experts): the waves' W_g steps during the K loop, reused for
// the cross-wave sums after it, plus the transpose tile of the scores.
template <int KW, int RT, int NT = 4>
constexpr size_t router_fused_lds() {
  constexpr int kEt = 16 * NT;
  constexpr size_t w = (size_t)KW * 32 * (kEt + 8) * 2;
  constexpr size_t r = (size_t)KW * 16 * RT * (kEt + 4) * 4;
  return (w > r ? w : r) + (size_t)16 * RT * (kEt + 1) * 4;
}

template <int KW, int RT, int AHEAD, int NT = 4>
__global__ __launch_bounds__(64 * KW, KW <= 4 ? 2 : 1) void router_fused_bf16_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ Wg, int n, int d, int E,
    const float* __restrict__ offset, const float* __restrict__ noise, float noise_std, int score,
    float* __restrict__ logits, float* __restrict__ scores, float* __restrict__ scores_t) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) char router_lds[];
  constexpr int kRows = 16 * RT;
  constexpr int kEt = 16 * NT;                          // experts per workgroup (expert tile)
  constexpr int kLdw = kEt + 8;                         // bf16 per LDS row of a W_g step
  constexpr int kRedLd = kEt + 4;                       // floats per LDS row of the cross-wave sums
  constexpr size_t kMain = router_fused_lds<KW, RT, NT>() - (size_t)kRows * (kEt + 1) * 4;
  bf16_t* sW = reinterpret_cast<bf16_t*>(router_lds);   // [KW][32][kLdw], during the K loop
  float* red = reinterpret_cast<float*>(router_lds);    // [KW][kRows][kRedLd], after it
  float* sT = reinterpret_cast<float*>(router_lds + kMain);   // [kRows][E + 1]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = blockIdx.x * kRows;
  const int e0 = blockIdx.y * kEt;                      // first expert of this workgroup's tile
  const int et = min(kEt, E - e0);                      // its experts
  const int ksl = d / KW;
  const int kbeg = wave * ksl;
  const int ns = ksl / 32;
  const int kl = (lane >> 4) << 3;
  // Buffer loads: the uniform part of every address (workgroup rows, wave
  // K slice, step) is in the resource base or the scalar offset, the lane
  // part in one 32-bit register.  X rows past n lie outside the resource
  // and read as zero.
  const __amdgpu_buffer_rsrc_t xr_src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(X + (size_t)r0 * d + kbeg), (short)0, min(kRows, n - r0) * d * 2, 0x00020000);
  int xoff[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) xoff[i] = ((16 * i + (lane & 15)) * d + kl) * 2;
  // W_g step loads, NT 16-byte chunks per lane: chunk lane + 64 h is row
  // kRstep h + lane / kCpr, experts e0 + 8 (lane % kCpr) .. +7 of the tile
  // (clamped to the last whole chunk of W_g past E; those LDS columns are
  // never read)
  constexpr int kCpr = kEt / 8;                         // 16-byte chunks per W_g row of the tile
  constexpr int kRstep = 64 / kCpr;                     // rows per chunk round
  const int wr = lane / kCpr, wc = (lane % kCpr) << 3;
  const __amdgpu_buffer_rsrc_t wr_src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(Wg + (size_t)kbeg * E), (short)0, ksl * E * 2, 0x00020000);
  const int woff = (wr * E + min(e0 + wc, E - 8)) * 2;
  bf16_t* sw = sW + wave * 32 * kLdw;
  const int tr_off = (8 * (lane >> 4) + ((lane >> 2) & 3)) * kLdw + 4 * (lane & 3);

  // Always NT 16-expert tiles: past E the extra tiles multiply LDS columns
  // of clamped copies and their sums are never read.
  f32x4_t acc[RT][NT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16x8_t xr[AHEAD][RT];
  u32x4_t wv[AHEAD][NT];
  auto load = [&](int st, int q) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
      xr[q][i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(xr_src, xoff[i], st * 64, 0));
#pragma unroll
    for (int h = 0; h < NT; ++h)
      wv[q][h] = __builtin_amdgcn_raw_buffer_load_b128(wr_src, woff, (st * 32 + kRstep * h) * E * 2, 0);
  };
  // AHEAD divides ns, so every round of the ring runs whole; loads are
  // issued unconditionally (the last round re-reads step ns - 1), which
  // keeps the loop free of branches.
#pragma unroll
  for (int q = 0; q < AHEAD; ++q) load(min(q, ns - 1), q);
  for (int st0 = 0; st0 < ns; st0 += AHEAD) {
#pragma unroll
    for (int q = 0; q < AHEAD; ++q) {
      // one wave's LDS operations execute in order: these stores land after
      // the previous step's transpose reads
#pragma unroll
      for (int h = 0; h < NT; ++h) *reinterpret_cast<u32x4_t*>(sw + (kRstep * h + wr) * kLdw + wc) = wv[q][h];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sw + tr_off + 16 * j));
        const v4i16 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sw + tr_off + 4 * kLdw + 16 * j));
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int i = 0; i < RT; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[q][i], b, acc[i][j], 0, 0, 0);
      }
      load(min(st0 + q + AHEAD, ns - 1), q);
    }
  }
  __syncthreads();   // every wave is done with its W_g rows; the sums reuse the space
  // C fragment: lane holds column (lane % 16), rows 4 (lane / 16) + r
  float* rw = red + wave * kRows * kRedLd;
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rw[(16 * i + 4 * (lane >> 4) + r) * kRedLd + 16 * j + (lane & 15)] = acc[i][j][r];
  __syncthreads();
  // Rows finish one per wave: lane l holds tile experts l + 64 jj.  A softmax
  // needs the whole row, so it runs only on workgroups that hold every
  // expert (the launcher keeps the expert tile at E); the per-expert scores
  // need no other expert.
  constexpr int kJ = (kEt + 63) / 64;
  constexpr int ld = kEt + 1;                           // odd stride: conflict-free both ways
  for (int rr = wave; rr < kRows; rr += KW) {
    const int row = r0 + rr;
    if (row >= n) break;
    float z[kJ];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int e = lane + 64 * jj;
      z[jj] = 0.f;
      if (e < et) {
        float v = red[rr * kRedLd + e];
#pragma unroll
        for (int w = 1; w < KW; ++w) v = v + red[(w * kRows + rr) * kRedLd + e];
        if (offset) v = v + offset[e0 + e];
        if (noise) v = v + noise_std * noise[(size_t)row * E + e0 + e];
        z[jj] = v;
        if (logits) logits[(size_t)row * E + e0 + e] = v;
      }
    }
    if (!scores && !scores_t) continue;
    float p[kJ];
    row_scores(z, kJ, et, score, p);
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int e = lane + 64 * jj;
      if (e < et) {
        if (scores) scores[(size_t)row * E + e0 + e] = p[jj];
        if (scores_t) sT[rr * ld + e] = p[jj];
      }
    }
  }
  if (!scores_t) return;
  __syncthreads();
  const int rows = min(kRows, n - r0);
  for (int item = tid; item < et * kRows; item += 64 * KW) {
    const int e = item / kRows, rr = item % kRows;
    if (rr < rows) scores_t[(size_t)(e0 + e) * n + r0 + rr] = sT[rr * ld + e];
  }
}

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
    row_scores(z, nj, E, score, p);
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

// Fused path, K in 32-wide steps per wave.
//  - Up to 64 experts (NT = 4, the workgroup holds all of them): RT = 2 when
//    there are at least 512 16-row tiles, else 1; MOE_ROUTER_KW_SMALL waves
//    per workgroup when there are fewer than 64 workgroups (short batches:
//    more K slices in flight), else MOE_ROUTER_KW_BIG.
//  - 65 to 128 experts (NT = 8, all experts in one workgroup, so softmax
//    rows stay whole): 4 waves, RT = 2.
//  - More experts with a per-expert score (sigmoid, sqrtsoftplus): 64-expert
//    tiles across workgroups (blockIdx.y), 4 waves, RT = 4 (or less when
//    that leaves fewer than 256 workgroups).
// Softmax rows over more than 128 experts take the split-K path.
struct FusedShape {
  bool ok;
  int kw, rt, nt, etiles;
};
static FusedShape router_fused_shape(int n, int d, int E, int dtype, int score) {
  FusedShape f{false, MOE_ROUTER_KW_BIG, 1, 4, 1};
  if (dtype != 1 || E % 16 != 0 || n < 1) return f;
  const int tiles = (n + 15) / 16;
  if (E <= 64) {
    f.rt = tiles >= 512 ? 2 : 1;
    const int blocks = (n + 16 * f.rt - 1) / (16 * f.rt);
    f.kw = blocks < 64 && d % (32 * MOE_ROUTER_KW_SMALL) == 0 ? MOE_ROUTER_KW_SMALL : MOE_ROUTER_KW_BIG;
  } else if (E <= 128 && (score == 0 || E % 64 != 0)) {
    f.kw = 4;
    f.rt = 2;
    f.nt = 8;
  } else if (score != 0) {
    f.kw = 4;
    f.nt = 4;
    f.etiles = (E + 63) / 64;
    f.rt = 4;
    while (f.rt > 1 && ((n + 16 * f.rt - 1) / (16 * f.rt)) * f.etiles < 256) f.rt /= 2;
  } else {
    return f;
  }
  f.ok = d % (32 * f.kw) == 0;
  return f;
}

// Workgroups with more than 64 KB of LDS need the kernel's limit raised;
// once per kernel, not per launch (the call costs host time).
template <auto kKernel, size_t kLds>
static hipError_t lds_limit_once() {
  if (kLds <= 65536) return hipSuccess;
  static const hipError_t status = hipFuncSetAttribute(reinterpret_cast<const void*>(kKernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)kLds);
  return status;
}

size_t router_workspace_bytes(int n, int d, int E, int dtype, int score) {
  if (router_fused_shape(n, d, E, dtype, score).ok) return 0;
  if (!router_uses_mfma(dtype, d, E)) return 0;
  const int s = router_splits(n, d, E);
  return s > 1 ? (size_t)s * n * E * sizeof(float) : 0;
}

hipError_t launch_router(const void* X, const void* Wg, int dtype, const float* offset,
                         const float* noise, float noise_std, int n, int d, int E, int score,
                         float* logits, float* scores, float* scores_t, void* ws, hipStream_t stream) {
  const FusedShape fs = router_fused_shape(n, d, E, dtype, score);
  if (fs.ok) {
    const bf16_t* x = static_cast<const bf16_t*>(X);
    const bf16_t* w = static_cast<const bf16_t*>(Wg);
    // the transpose tile at the end of the LDS only when scores_t is
    // requested: without it two workgroups fit on a CU
    auto go = [&](auto kern, hipError_t limit, size_t lds, int rows, int threads) -> hipError_t {
      if (limit != hipSuccess) return limit;
      const size_t lds_used = scores_t ? lds : lds - (size_t)rows * (16 * fs.nt + 1) * 4;
      hipLaunchKernelGGL(kern, dim3((unsigned)((n + rows - 1) / rows), fs.etiles), dim3(threads), lds_used, stream,
                         x, w, n, d, E, offset, noise, noise_std, score, logits, scores, scores_t);
      return hipGetLastError();
    };
#define MOE_FUSED(KW, RT, A, NT)                                                                         \
  go(router_fused_bf16_kernel<KW, RT, A, NT>,                                                            \
     lds_limit_once<router_fused_bf16_kernel<KW, RT, A, NT>, router_fused_lds<KW, RT, NT>()>(),           \
     router_fused_lds<KW, RT, NT>(), 16 * RT, 64 * KW)
#define MOE_FUSED_RING(KW, RT, NT)                                                                    \
  (ns % kFusedAhead == 0 ? MOE_FUSED(KW, RT, kFusedAhead, NT) : ns % 2 == 0 ? MOE_FUSED(KW, RT, 2, NT) \
                                                                           : MOE_FUSED(KW, RT, 1, NT))
    const int ns = d / fs.kw / 32;   // K steps per wave
    hipError_t err;
    if (fs.nt == 8) err = ns % 2 == 0 ? MOE_FUSED(4, 2, 2, 8) : MOE_FUSED(4, 2, 1, 8);
    else if (fs.etiles > 1 && fs.rt == 4) err = MOE_FUSED_RING(4, 4, 4);
    else if (fs.etiles > 1 && fs.rt == 2) err = MOE_FUSED_RING(4, 2, 4);
    else if (fs.etiles > 1) err = MOE_FUSED_RING(4, 1, 4);
    else if (fs.kw == MOE_ROUTER_KW_SMALL && MOE_ROUTER_KW_SMALL != MOE_ROUTER_KW_BIG) err = MOE_FUSED_RING(MOE_ROUTER_KW_SMALL, 1, 4);
    else if (fs.rt == 2) err = MOE_FUSED_RING(MOE_ROUTER_KW_BIG, 2, 4);
    else err = MOE_FUSED_RING(MOE_ROUTER_KW_BIG, 1, 4);
#undef MOE_FUSED_RING
#undef MOE_FUSED
    return err;
  }
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
