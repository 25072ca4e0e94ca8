// Dispatch (gather into the expert-major buffer) and combine (gate-weighted
// sum back to token order).
//
// MoE-routing pages: page 2 "Expert choice routing", section "The math":
// X_in[e] = P[e] X with P = onehot(I), Y[e] = G[e] * Expert_e(X_in[e]),
// out = scatter_add(Y, I); page 1 "Token choice vs expert choice routing",
// section "Dropped tokens flow in opposite directions" (a dropped token
// passes through on the residual); page 5 "MoE routing strategies
// explained", strategy 3 (the always-on shared expert is added for every
// token).
//
// Both kernels are pure HBM streams: one wave per row, 16-byte loads and
// stores, every byte read or written once.  Each wave issues all the loads
// of a row (or of a batch of rows) before it consumes any, so one memory
// round trip covers them.  The combine is a gather rather than a scatter:
// each token walks its own slot list in a fixed order and accumulates in
// fp32, so there are no floating-point atomics and the result is bitwise
// reproducible.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCopyUnroll = 8;   // 16-byte chunks per lane in flight (8 KB per wave)

__global__ __launch_bounds__(256) void dispatch_vec_kernel(const char* __restrict__ X, int64_t row_bytes,
                                                           const int32_t* __restrict__ slot_token,
                                                           const int32_t* __restrict__ n_kept,
                                                           int64_t M_max, char* __restrict__ Xp) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = min((int64_t)*n_kept, M_max);
  if (row >= rows) return;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(X + (int64_t)slot_token[row] * row_bytes);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(Xp + row * row_bytes);
  const int64_t nv = row_bytes / 16;
  for (int64_t base = 0; base < nv; base += 64 * kCopyUnroll) {
    u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * 64 + lane;
      if (i < nv) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * 64 + lane;
      if (i < nv) dst[i] = v[u];
    }
  }
}

template <typename V>
__global__ __launch_bounds__(256) void dispatch_kernel(const char* __restrict__ X, int64_t row_bytes,
                                                       const int32_t* __restrict__ slot_token,
                                                       const int32_t* __restrict__ n_kept,
                                                       int64_t M_max, char* __restrict__ Xp) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = min((int64_t)*n_kept, M_max);
  if (row >= rows) return;
  const V* src = reinterpret_cast<const V*>(X + (int64_t)slot_token[row] * row_bytes);
  V* dst = reinterpret_cast<V*>(Xp + row * row_bytes);
  const int64_t nv = row_bytes / (int64_t)sizeof(V);
  for (int64_t i = lane; i < nv; i += 64) dst[i] = src[i];
}

hipError_t launch_dispatch(const void* X, int elem_bytes, int n, int d, const int32_t* slot_token,
                           const int32_t* n_kept, int64_t M_max, void* X_perm, hipStream_t stream) {
  (void)n;
  const int64_t row_bytes = (int64_t)d * elem_bytes;
  const dim3 grid((unsigned)((M_max + 3) / 4)), block(256);
  const char* src = static_cast<const char*>(X);
  char* dst = static_cast<char*>(X_perm);
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(dispatch_vec_kernel, grid, block, 0, stream, src, row_bytes, slot_token, n_kept,
                       M_max, dst);
  else if (row_bytes % 4 == 0)
    hipLaunchKernelGGL(dispatch_kernel<uint32_t>, grid, block, 0, stream, src, row_bytes, slot_token,
                       n_kept, M_max, dst);
  else
    hipLaunchKernelGGL(dispatch_kernel<uint16_t>, grid, block, 0, stream, src, row_bytes, slot_token,
                       n_kept, M_max, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine

// 16 bytes of a row: 4 fp32 or 8 bf16 values.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  MOE_DEV static void unpack(const u32x4_t& r, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
  }
  MOE_DEV static u32x4_t pack(const float* v) {
    return u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                   __float_as_uint(v[3])};
  }
  MOE_DEV static float one(const float* p) { return *p; }
  MOE_DEV static void put(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  MOE_DEV static void unpack(const u32x4_t& r, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
  MOE_DEV static u32x4_t pack(const float* v) {
    return u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
  }
  MOE_DEV static float one(const bf16_t* p) { return bf16_to_f32(*p); }
  MOE_DEV static void put(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// One wave per token.  acc = residual; acc += shared; then acc += g * y for
// the token's slots in list order (negative entries are dropped
// assignments; slot_gate NULL: every g = 1, the dispatch's backward); one
// rounding at the store.  The token index is uniform
// across the wave, so its list bounds, slot ids and gates are scalar loads:
// they run beside the vector loads of the residual row instead of queueing
// behind them (vector loads complete in issue order).  Per column pass: the
// residual and shared rows are requested, then the first kSlotBatch list
// entries and their gates, then those slots' rows; only then is the
// residual unpacked, so its fetch, the list lookups and the first rows'
// fetch overlap.  Later batches follow one at a time.
#ifndef MOE_COMBINE_CHUNKS
#define MOE_COMBINE_CHUNKS 4
#endif
#ifndef MOE_COMBINE_BATCH
#define MOE_COMBINE_BATCH 2
#endif
constexpr int kChunks = MOE_COMBINE_CHUNKS;     // 16-byte chunks per lane per column pass
constexpr int kSlotBatch = MOE_COMBINE_BATCH;   // expert rows in flight per wave

template <typename T, bool kRes, bool kShared>
__global__ __launch_bounds__(256) void combine_vec_kernel(const T* __restrict__ Y,
                                                          const int32_t* __restrict__ token_offset,
                                                          const int32_t* __restrict__ token_slot,
                                                          const float* __restrict__ slot_gate, int n,
                                                          int d, const T* __restrict__ residual,
                                                          const T* __restrict__ shared,
                                                          T* __restrict__ out) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= n) return;
  const size_t rowoff = (size_t)t * d;
  const int q0 = token_offset[t], q1 = token_offset[t + 1];
  for (int col0 = 0; col0 < d; col0 += 64 * V * kChunks) {
    // Columns past d (a ragged last pass) load the row's last chunk instead
    // and are not stored: no load sits behind a per-lane branch, which would
    // make the compiler wait for every earlier load first.
    bool ok[kChunks];
    int cl[kChunks];
    u32x4_t rres[kChunks], rsh[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int col = col0 + (c * 64 + lane) * V;
      ok[c] = col < d;
      cl[c] = min(col, d - V);
      if (kRes) rres[c] = *reinterpret_cast<const u32x4_t*>(residual + rowoff + cl[c]);
      if (kShared) rsh[c] = *reinterpret_cast<const u32x4_t*>(shared + rowoff + cl[c]);
    }
    int sl[kSlotBatch];
    float gl[kSlotBatch];
    u32x4_t ry[kSlotBatch][kChunks];
    auto fetch = [&](int qb) {
#pragma unroll
      for (int b = 0; b < kSlotBatch; ++b) sl[b] = qb + b < q1 ? token_slot[qb + b] : -1;
#pragma unroll
      for (int b = 0; b < kSlotBatch; ++b) gl[b] = sl[b] < 0 ? 0.f : slot_gate ? slot_gate[sl[b]] : 1.f;
      // entries past the list (or dropped) load row 0, which always exists,
      // and are skipped when adding
#pragma unroll
      for (int b = 0; b < kSlotBatch; ++b) {
        const T* yrow = Y + (size_t)(sl[b] < 0 ? 0 : sl[b]) * d;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) ry[b][c] = *reinterpret_cast<const u32x4_t*>(yrow + cl[c]);
      }
    };
    float acc[kChunks][V];
    auto add = [&]() {
#pragma unroll
      for (int b = 0; b < kSlotBatch; ++b) {
        if (sl[b] < 0) continue;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          float y[V];
          Elem<T>::unpack(ry[b][c], y);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[c][i] = fmaf(gl[b], y[i], acc[c][i]);
        }
      }
    };
    fetch(q0);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (kRes) {
        Elem<T>::unpack(rres[c], acc[c]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) acc[c][i] = 0.f;
      }
      if (kShared) {
        float sh[V];
        Elem<T>::unpack(rsh[c], sh);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[c][i] += sh[i];
      }
    }
    add();
    for (int qb = q0 + kSlotBatch; qb < q1; qb += kSlotBatch) {
      fetch(qb);
      add();
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      if (ok[c])
        *reinterpret_cast<u32x4_t*>(out + rowoff + col0 + (c * 64 + lane) * V) = Elem<T>::pack(acc[c]);
  }
}

// Scalar path for rows that are not a whole number of 16-byte chunks.
template <typename T>
__global__ __launch_bounds__(256) void combine_scalar_kernel(const T* __restrict__ Y,
                                                             const int32_t* __restrict__ token_offset,
                                                             const int32_t* __restrict__ token_slot,
                                                             const float* __restrict__ slot_gate, int n,
                                                             int d, const T* __restrict__ residual,
                                                             const T* __restrict__ shared,
                                                             T* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  const int q0 = token_offset[t], q1 = token_offset[t + 1];
  const size_t rowoff = (size_t)t * d;
  for (int c = lane; c < d; c += 64) {
    float a = residual ? Elem<T>::one(residual + rowoff + c) : 0.f;
    if (shared) a += Elem<T>::one(shared + rowoff + c);
    for (int q = q0; q < q1; ++q) {
      const int s = token_slot[q];
      if (s < 0) continue;
      a = fmaf(slot_gate ? slot_gate[s] : 1.f, Elem<T>::one(Y + (size_t)s * d + c), a);
    }
    Elem<T>::put(out + rowoff + c, a);
  }
}

template <typename T>
static hipError_t launch_combine_t(const T* Y, const int32_t* token_offset, const int32_t* token_slot,
                                   const float* slot_gate, int n, int d, const T* residual, const T* shared,
                                   T* out, hipStream_t stream) {
  const dim3 grid((n + 3) / 4), block(256);
  constexpr int V = Elem<T>::kVec;
  if (d % V != 0) {
    hipLaunchKernelGGL(combine_scalar_kernel<T>, grid, block, 0, stream, Y, token_offset, token_slot, slot_gate,
                       n, d, residual, shared, out);
  } else {
    auto k = residual ? (shared ? combine_vec_kernel<T, true, true> : combine_vec_kernel<T, true, false>)
                      : (shared ? combine_vec_kernel<T, false, true> : combine_vec_kernel<T, false, false>);
    hipLaunchKernelGGL(k, grid, block, 0, stream, Y, token_offset, token_slot, slot_gate, n, d, residual, shared,
                       out);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* Y, int dtype, const int32_t* token_offset,
                          const int32_t* token_slot, const float* slot_gate, int n, int d,
                          const void* residual, const void* shared, void* out, hipStream_t stream) {
  if (dtype == 1)
    return launch_combine_t(static_cast<const bf16_t*>(Y), token_offset, token_slot, slot_gate, n, d,
                            static_cast<const bf16_t*>(residual), static_cast<const bf16_t*>(shared),
                            static_cast<bf16_t*>(out), stream);
  return launch_combine_t(static_cast<const float*>(Y), token_offset, token_slot, slot_gate, n, d,
                          static_cast<const float*>(residual), static_cast<const float*>(shared),
                          static_cast<float*>(out), stream);
}

}  // namespace moe
