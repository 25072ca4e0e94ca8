// Routing map: per-expert counts and offsets, the capacity rule in token
// arrival order, the expert-major slot table, and the token-side lists the
// combine walks.
//
// MoE-routing pages: page 1 "Token choice vs expert choice routing",
// section "Dropped tokens flow in opposite directions" (a fixed per-expert
// buffer; an assignment reaching it when full is not computed and its token
// keeps the residual; dropless computes every assignment); page 5 "MoE
// routing strategies explained", strategy 2 (tokens beyond capacity bypass
// the expert by way of the residual); page 2 "Expert choice routing", section "The
// math" (P = onehot(I): slot e*k + j carries token I[e, j]).
//
// Token choice runs as a stable counting sort of the n*k arrivals by expert.
// Arrival a is assignment (t, r) = (a / k, a % k) in token-major order, or
// (a % n, a / n) in rank-major order (every first choice before any second
// one):
//  1. chunk histograms (LDS integer atomics; counts are order-free),
//  2. one workgroup turns them into per-chunk starting positions per expert
//     (a scan over chunks in chunk order) and expert offsets of the kept
//     rows (a scan over experts),
//  3. one workgroup per chunk, one wave per 64 consecutive arrivals: lanes
//     with the same expert find each other with one ballot per expert-id
//     bit, their rank inside the wave is a popcount, each wave's count per
//     expert goes to LDS, and a scan over the waves in order (thread e for
//     expert e) gives every wave its experts' starting positions.  A
//     position below the capacity is kept; its slot is offset[e] + position.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kMapChunk = 1024;      // arrivals per chunk
constexpr int kScanThreads = 1024;

// Element of idx [n, k] that arrives a-th.
MOE_DEV int64_t arrival_elem(int64_t a, int n, int k, int rank_major) {
  return rank_major ? (a % n) * k + a / n : a;
}

__global__ __launch_bounds__(256) void map_chunk_hist_kernel(const int32_t* __restrict__ idx,
                                                             int64_t M, int n, int k, int E,
                                                             int rank_major,
                                                             int32_t* __restrict__ chunk_hist) {
  extern __shared__ int sh[];
  for (int e = threadIdx.x; e < E; e += 256) sh[e] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kMapChunk;
  for (int i = threadIdx.x; i < kMapChunk; i += 256) {
    const int64_t a = a0 + i;
    if (a < M) {
      const int e = idx[arrival_elem(a, n, k, rank_major)];
      if ((unsigned)e < (unsigned)E) atomicAdd(&sh[e], 1);   // out-of-range ids are dropped
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_hist[(size_t)blockIdx.x * E + e] = sh[e];
}

// One workgroup: thread e scans expert e's chunk counts in chunk order; then
// a workgroup scan over experts of the kept counts gives the slot offsets.
// The counts are loaded kScanBatch chunks at a time, every load from a
// clamped address and issued before the first add, so a batch costs one
// memory latency rather than one per chunk.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(kScanThreads) void map_scan_kernel(
    const int32_t* __restrict__ chunk_hist, int nchunks, int E, int capacity,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ expert_count,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ n_kept) {
  __shared__ int scratch[kScanThreads / 64];
  const int e = threadIdx.x;
  int kept = 0;
  if (e < E) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) v[u] = chunk_hist[(size_t)min(c0 + u, nchunks - 1) * E + e];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (c0 + u < nchunks) {
          chunk_base[(size_t)(c0 + u) * E + e] = run;
          run += v[u];
        }
      }
    }
    expert_count[e] = run;
    kept = capacity < 0 ? run : min(run, capacity);
  }
  int total = 0;
  const int off = block_exclusive_scan<kScanThreads>(kept, scratch, &total);
  if (e < E) expert_offset[e] = off;
  if (e == 0) {
    expert_offset[E] = total;
    *n_kept = total;
  }
}

// Token choice also writes the token-side lists: token t's entries are its
// k assignments in rank order (token_offset[t] = t*k), -1 for a dropped one.
// Wave w of chunk c takes arrivals c*kMapChunk + 64 w + lane, one per lane.
// kSingle: the whole batch is one chunk (n k <= kMapChunk, decode-sized
// batches), and this one workgroup also does the histogram and scans of
// steps 1 and 2: the chunk starts every expert at 0, the per-expert totals
// are its counts, and a workgroup scan of the kept counts gives the
// offsets.  One launch instead of three, with the same slots.
constexpr int kScatterWaves = kMapChunk / 64;

template <bool kSingle>
__global__ __launch_bounds__(kMapChunk) void map_scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ gate, int64_t M, int n, int k, int E,
    int rank_major, int nbits, int capacity, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ expert_offset, MapPtrs m) {
  extern __shared__ int sm[];                       // [kScatterWaves][E] wave counts, then [E] offsets
  int* eoff = sm + kScatterWaves * E;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < kScatterWaves * E; i += kMapChunk) sm[i] = 0;
  if (!kSingle)
    for (int e = threadIdx.x; e < E; e += kMapChunk) eoff[e] = expert_offset[e];
  // 32-bit indices (the host checks n k < 2^31): a 64-bit division per
  // element would cost more than the rest of the work
  const int Mi = (int)M;
  const int a = c * kMapChunk + 64 * w + lane;
  const bool inrange = a < Mi;
  const int q = inrange ? (rank_major ? (a % n) * k + a / n : a) : 0;   // element of idx arriving a-th
  const int e_raw = inrange ? idx[q] : 0;
  const float g = inrange ? gate[q] : 0.f;
  const bool valid = inrange && (unsigned)e_raw < (unsigned)E;
  const int e = valid ? e_raw : 0;
  // lanes of this wave with the same expert, and this lane's rank among them
  uint64_t match = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    match &= bit ? bal : ~bal;
  }
  const int rank = __popcll(match & ((1ull << lane) - 1ull));
  __syncthreads();                                  // counts cleared, offsets staged
  if (valid && (match >> lane) == 1ull) sm[w * E + e] = __popcll(match);   // the expert's last lane
  __syncthreads();
  // thread x < E: expert x's running position through the waves in order,
  // from the chunk's starting position
  int kept = 0;
  if ((int)threadIdx.x < E) {
    int run = kSingle ? 0 : chunk_base[(size_t)c * E + threadIdx.x];
#pragma unroll
    for (int v = 0; v < kScatterWaves; ++v) {
      const int cnt = sm[v * E + threadIdx.x];
      sm[v * E + threadIdx.x] = run;
      run += cnt;
    }
    if (kSingle) {
      m.expert_count[threadIdx.x] = run;
      kept = capacity < 0 ? run : min(run, capacity);
    }
  }
  if (kSingle) {
    __shared__ int scratch[kMapChunk / 64];
    int total = 0;
    const int off = block_exclusive_scan<kMapChunk>(kept, scratch, &total);
    if ((int)threadIdx.x < E) {
      eoff[threadIdx.x] = off;
      m.expert_offset[threadIdx.x] = off;
    }
    if (threadIdx.x == 0) {
      m.expert_offset[E] = total;
      *m.n_kept = total;
    }
  }
  __syncthreads();
  if (c == 0 && threadIdx.x == 0) m.token_offset[Mi / k] = Mi;
  if (inrange) {
    const int pos = valid ? sm[w * E + e] + rank : 0;
    int32_t s = -1;
    if (valid && (capacity < 0 || pos < capacity)) {
      s = eoff[e] + pos;
      m.slot_token[s] = q / k;
      m.slot_gate[s] = g;
    }
    m.assign_slot[q] = s;
    m.token_slot[q] = s;
    if (q % k == 0) m.token_offset[q / k] = (int32_t)q;
  }
}

// ---------------------------------------------------------------- expert choice
// Token t's list holds the slots of the experts that picked it, in
// ascending expert order.  A bit mask [n][ceil(E/32)] records who picked
// whom (integer atomics, order-free); a token's list length is the popcount
// of its row, the offsets are a workgroup scan, and the position of (t, e)
// in t's list is the popcount of t's bits below e.

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t count,
                                                       uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) p[i] = v;
}

__global__ __launch_bounds__(256) void ec_slots_kernel(const int32_t* __restrict__ I,
                                                       const float* __restrict__ G, int n, int E, int k,
                                                       int W, MapPtrs m, uint32_t* __restrict__ mask) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= (int64_t)E * k) return;
  const int e = (int)(s / k);
  const int t = I[s];
  m.slot_token[s] = t;
  m.slot_gate[s] = G[s];
  m.assign_slot[s] = (int32_t)s;
  if ((unsigned)t < (unsigned)n) atomicOr(&mask[(size_t)t * W + (e >> 5)], 1u << (e & 31));
  if (s - (int64_t)e * k == 0) {
    m.expert_count[e] = k;
    m.expert_offset[e] = e * k;
    if (e == E - 1) {
      m.expert_offset[E] = E * k;
      *m.n_kept = E * k;
    }
  }
}

// One workgroup turns the mask into token offsets, kTokPer tokens per thread
// per pass: each pass loads all its mask words at once, scans the counts
// across the workgroup and carries the running total to the next pass.
constexpr int kTokPer = 4;

__global__ __launch_bounds__(kScanThreads) void ec_token_offsets_kernel(
    const uint32_t* __restrict__ mask, int n, int W, int32_t* __restrict__ token_offset) {
  __shared__ int scratch[kScanThreads / 64];
  int carry = 0;
  for (int base = 0; base < n; base += kScanThreads * kTokPer) {
    const int t0 = base + threadIdx.x * kTokPer;
    int cnt[kTokPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kTokPer; ++i) {
      const int t = t0 + i;
      int c = 0;
      if (t < n)
        for (int w = 0; w < W; ++w) c += __popc(mask[(size_t)t * W + w]);
      cnt[i] = c;
      sum += c;
    }
    int total = 0;
    int run = carry + block_exclusive_scan<kScanThreads>(sum, scratch, &total);
#pragma unroll
    for (int i = 0; i < kTokPer; ++i) {
      if (t0 + i < n) token_offset[t0 + i] = run;
      run += cnt[i];
    }
    carry += total;
  }
  if (threadIdx.x == 0) token_offset[n] = carry;
}

__global__ __launch_bounds__(256) void ec_token_fill_kernel(const int32_t* __restrict__ I,
                                                            const uint32_t* __restrict__ mask,
                                                            const int32_t* __restrict__ token_offset,
                                                            int n, int E, int k, int W,
                                                            int32_t* __restrict__ token_slot) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= (int64_t)E * k) return;
  const int e = (int)(s / k);
  const int t = I[s];
  if ((unsigned)t >= (unsigned)n) return;
  const uint32_t* row = mask + (size_t)t * W;
  int before = 0;
  for (int w = 0; w < (e >> 5); ++w) before += __popc(row[w]);
  before += __popc(row[e >> 5] & ((1u << (e & 31)) - 1u));
  token_slot[token_offset[t] + before] = (int32_t)s;
}

// The whole map in one workgroup, for batches whose token mask and token
// offsets fit in LDS: every thread loads its slots' tokens and gates at
// once (slot u * 1024 + tid, u < kEcSmallSlots), builds the mask with LDS
// atomics, scans the popcounts in LDS and takes each slot's list position
// from the LDS mask, so only the loads of I, G and the result stores touch
// global memory, and nothing needs clearing between calls.  Same results
// as the four-kernel path.
constexpr int kEcSmallSlots = 16;
constexpr int kEcSmallLdsWords = 16384;   // 64 KB of mask and offsets

__global__ __launch_bounds__(kScanThreads) void ec_map_small_kernel(const int32_t* __restrict__ I,
                                                                    const float* __restrict__ G, int n,
                                                                    int E, int k, int W, MapPtrs m) {
  extern __shared__ uint32_t ec_lds[];
  uint32_t* smask = ec_lds;                                   // [n][W]
  int* soff = reinterpret_cast<int*>(ec_lds + (size_t)n * W);  // [n]
  __shared__ int scratch[kScanThreads / 64];
  const int tid = threadIdx.x;
  const int M = E * k;
  int tok[kEcSmallSlots];
  float gt[kEcSmallSlots];
#pragma unroll
  for (int u = 0; u < kEcSmallSlots; ++u) {
    const int s = u * kScanThreads + tid;
    tok[u] = s < M ? I[s] : -1;
    gt[u] = s < M ? G[s] : 0.f;
  }
  for (int i = tid; i < n * W; i += kScanThreads) smask[i] = 0u;
  if (tid < E) {
    m.expert_count[tid] = k;
    m.expert_offset[tid] = tid * k;
  }
  if (tid == 0) {
    m.expert_offset[E] = M;
    *m.n_kept = M;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kEcSmallSlots; ++u) {
    const int s = u * kScanThreads + tid;
    if (s < M) {
      const int t = tok[u];
      const int e = s / k;
      m.slot_token[s] = t;
      m.slot_gate[s] = gt[u];
      m.assign_slot[s] = s;
      if ((unsigned)t < (unsigned)n) atomicOr(&smask[t * W + (e >> 5)], 1u << (e & 31));
    }
  }
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < n; base += kScanThreads * kTokPer) {
    const int t0 = base + tid * kTokPer;
    int cnt[kTokPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kTokPer; ++i) {
      int c = 0;
      if (t0 + i < n)
        for (int w = 0; w < W; ++w) c += __popc(smask[(t0 + i) * W + w]);
      cnt[i] = c;
      sum += c;
    }
    int total = 0;
    int run = carry + block_exclusive_scan<kScanThreads>(sum, scratch, &total);
#pragma unroll
    for (int i = 0; i < kTokPer; ++i) {
      if (t0 + i < n) {
        soff[t0 + i] = run;
        m.token_offset[t0 + i] = run;
      }
      run += cnt[i];
    }
    carry += total;
  }
  if (tid == 0) m.token_offset[n] = carry;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kEcSmallSlots; ++u) {
    const int s = u * kScanThreads + tid;
    const int t = tok[u];
    if (s < M && (unsigned)t < (unsigned)n) {
      const int e = s / k;
      const uint32_t* row = smask + t * W;
      int before = 0;
      for (int w = 0; w < (e >> 5); ++w) before += __popc(row[w]);
      before += __popc(row[e >> 5] & ((1u << (e & 31)) - 1u));
      m.token_slot[soff[t] + before] = s;
    }
  }
}

// Expert choice with k = 0 (a batch too small for any expert to take a
// token): every count, offset and token list is empty.
__global__ __launch_bounds__(256) void ec_empty_map_kernel(int n, int E, MapPtrs m) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < E) m.expert_count[i] = 0;
  if (i <= E) m.expert_offset[i] = 0;
  if (i <= n) m.token_offset[i] = 0;
  if (i == 0) *m.n_kept = 0;
}

// ---------------------------------------------------------------- host side

static int chunks_of(int64_t M) { return (int)((M + kMapChunk - 1) / kMapChunk); }

size_t map_workspace_bytes(int dir, int n, int E, int k) {
  if (dir == 0) return (size_t)2 * chunks_of((int64_t)n * k) * E * sizeof(int32_t);
  return (size_t)n * ((E + 31) / 32) * sizeof(uint32_t);
}

hipError_t launch_build_map_tc(const int32_t* idx, const float* gate, int n, int E, int k,
                               int capacity, int rank_major, const MapPtrs& m, void* ws,
                               hipStream_t stream) {
  const int64_t M = (int64_t)n * k;
  const int nch = chunks_of(M);
  int32_t* chunk_hist = static_cast<int32_t*>(ws);
  int32_t* chunk_base = chunk_hist + (size_t)nch * E;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t lds = (kScatterWaves + 1) * E * sizeof(int);
  if (nch == 1) {
    hipLaunchKernelGGL(map_scatter_kernel<true>, dim3(1), dim3(kMapChunk), lds, stream, idx, gate, M, n, k, E,
                       rank_major, nbits, capacity, chunk_base, m.expert_offset, m);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(map_chunk_hist_kernel, dim3(nch), dim3(256), E * sizeof(int), stream, idx, M, n, k,
                     E, rank_major, chunk_hist);
  hipLaunchKernelGGL(map_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, chunk_hist, nch, E,
                     capacity, chunk_base, m.expert_count, m.expert_offset, m.n_kept);
  hipLaunchKernelGGL(map_scatter_kernel<false>, dim3(nch), dim3(kMapChunk), lds, stream, idx, gate, M, n, k, E,
                     rank_major, nbits, capacity, chunk_base, m.expert_offset, m);
  return hipGetLastError();
}

hipError_t launch_build_map_ec(const int32_t* I, const float* G, int n, int E, int k,
                               const MapPtrs& m, void* ws, hipStream_t stream) {
  if (k == 0) {
    hipLaunchKernelGGL(ec_empty_map_kernel, dim3((unsigned)((max(n, E) + 1 + 255) / 256)), dim3(256), 0,
                       stream, n, E, m);
    return hipGetLastError();
  }
  const int W = (E + 31) / 32;
  if ((int64_t)E * k <= (int64_t)kScanThreads * kEcSmallSlots &&
      (int64_t)n * (W + 1) <= kEcSmallLdsWords) {
    hipLaunchKernelGGL(ec_map_small_kernel, dim3(1), dim3(kScanThreads),
                       (size_t)n * (W + 1) * sizeof(uint32_t), stream, I, G, n, E, k, W, m);
    return hipGetLastError();
  }
  uint32_t* mask = static_cast<uint32_t*>(ws);
  const int64_t words = (int64_t)n * W;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                     mask, words, 0u);
  const int64_t M = (int64_t)E * k;
  const dim3 grid((unsigned)((M + 255) / 256));
  hipLaunchKernelGGL(ec_slots_kernel, grid, dim3(256), 0, stream, I, G, n, E, k, W, m, mask);
  hipLaunchKernelGGL(ec_token_offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, mask, n, W,
                     m.token_offset);
  hipLaunchKernelGGL(ec_token_fill_kernel, grid, dim3(256), 0, stream, I, mask, m.token_offset, n, E,
                     k, W, m.token_slot);
  return hipGetLastError();
}

}  // namespace moe
