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
// stores, every byte read or written once.  The combine is a gather rather
// than a scatter: each token walks its own slot list (token_offset /
// token_slot) in a fixed order and accumulates in fp32, so there are no
// floating-point atomics and the result is bitwise reproducible.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

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
    hipLaunchKernelGGL(dispatch_kernel<uint4>, grid, block, 0, stream, src, row_bytes, slot_token,
                       n_kept, M_max, dst);
  else if (row_bytes % 4 == 0)
    hipLaunchKernelGGL(dispatch_kernel<uint32_t>, grid, block, 0, stream, src, row_bytes, slot_token,
                       n_kept, M_max, dst);
  else
    hipLaunchKernelGGL(dispatch_kernel<uint16_t>, grid, block, 0, stream, src, row_bytes, slot_token,
                       n_kept, M_max, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;                       // elements per 16-byte access
  MOE_DEV static void load(const float* p, float* v) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  MOE_DEV static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
  MOE_DEV static float one(const float* p) { return *p; }
  MOE_DEV static void put(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  MOE_DEV static void load(const bf16_t* p, float* v) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  MOE_DEV static void store(bf16_t* p, const float* v) {
    uint4 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]);
    q.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = q;
  }
  MOE_DEV static float one(const bf16_t* p) { return bf16_to_f32(*p); }
  MOE_DEV static void put(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// One wave per token.  acc = residual; acc += shared; then acc += g * y for
// the token's slots in list order; one rounding at the store.
template <typename T, bool kVecPath>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ Y,
                                                      const int32_t* __restrict__ token_offset,
                                                      const int32_t* __restrict__ token_slot,
                                                      const float* __restrict__ slot_gate, int n,
                                                      int d, const T* __restrict__ residual,
                                                      const T* __restrict__ shared, T* __restrict__ out) {
  constexpr int V = kVecPath ? Elem<T>::kVec : 1;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  const int q0 = token_offset[t], q1 = token_offset[t + 1];
  const size_t rowoff = (size_t)t * d;
  for (int c = lane * V; c < d; c += 64 * V) {
    float acc[V];
    if (kVecPath) {
      if (residual) {
        Elem<T>::load(residual + rowoff + c, acc);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;
      }
      if (shared) {
        float s[V];
        Elem<T>::load(shared + rowoff + c, s);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += s[i];
      }
      for (int q = q0; q < q1; ++q) {
        const int s = token_slot[q];
        const float g = slot_gate[s];
        float y[V];
        Elem<T>::load(Y + (size_t)s * d + c, y);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(g, y[i], acc[i]);
      }
      Elem<T>::store(out + rowoff + c, acc);
    } else {
      float a = residual ? Elem<T>::one(residual + rowoff + c) : 0.f;
      if (shared) a += Elem<T>::one(shared + rowoff + c);
      for (int q = q0; q < q1; ++q) {
        const int s = token_slot[q];
        a = fmaf(slot_gate[s], Elem<T>::one(Y + (size_t)s * d + c), a);
      }
      Elem<T>::put(out + rowoff + c, a);
    }
  }
}

hipError_t launch_combine(const void* Y, int dtype, const int32_t* token_offset,
                          const int32_t* token_slot, const float* slot_gate, int n, int d,
                          const void* residual, const void* shared, void* out, hipStream_t stream) {
  const dim3 grid((n + 3) / 4), block(256);
  if (dtype == 1) {
    typedef bf16_t T;
    const bool vec = d % 8 == 0;
    auto k = vec ? combine_kernel<T, true> : combine_kernel<T, false>;
    hipLaunchKernelGGL(k, grid, block, 0, stream, static_cast<const T*>(Y), token_offset, token_slot,
                       slot_gate, n, d, static_cast<const T*>(residual),
                       static_cast<const T*>(shared), static_cast<T*>(out));
  } else {
    typedef float T;
    const bool vec = d % 4 == 0;
    auto k = vec ? combine_kernel<T, true> : combine_kernel<T, false>;
    hipLaunchKernelGGL(k, grid, block, 0, stream, static_cast<const T*>(Y), token_offset, token_slot,
                       slot_gate, n, d, static_cast<const T*>(residual),
                       static_cast<const T*>(shared), static_cast<T*>(out));
  }
  return hipGetLastError();
}

}  // namespace moe
