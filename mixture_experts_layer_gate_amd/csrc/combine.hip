// Weighted combine: out[t] = sum_{j ascending} w[t][j] * y_sorted[inv_perm[t*k + j]],
// plus, for shared (always-active) experts, y[T*k + s*T + t] for s ascending.
//
// The final top-k sum is its own step after the expert FFN (MegaFlux,
// section 2.1); token identity, slot and weight of every assignment are kept
// for it (MegaFlux, appendix A.2). One block per token; each thread owns
// 8 consecutive columns (one 16-byte bf16 vector), accumulates in fp32 and
// stores with round-to-nearest-even.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombThreads = 256;

template <int kDtype>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const void* __restrict__ y,
                                                               const int32_t* __restrict__ inv_perm,
                                                               const float* __restrict__ w,
                                                               void* __restrict__ out, int64_t d,
                                                               int k, int64_t n_assign, int n_shared,
                                                               int64_t T) {
  const int64_t t = blockIdx.x;
  const int64_t nvec = d / 8;
  for (int64_t c = threadIdx.x; c < nvec; c += kCombThreads) {
    float acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
    for (int j = 0; j < k; ++j) {
      int64_t p = inv_perm[t * k + j];
      p = p < 0 ? 0 : (p >= n_assign ? n_assign - 1 : p);
      const float wj = w[t * k + j];
      float v[8];
      if constexpr (kDtype == 1) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(y) + p * d + c * 8);
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
      } else {
        const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(y) + p * d + c * 8);
        const float4 a = q[0], b = q[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = __builtin_fmaf(wj, v[r], acc[r]);
    }
    // shared experts: rows n_assign + s*T + t, weight 1, after the routed slots
    for (int sh = 0; sh < n_shared; ++sh) {
      const int64_t p = n_assign + static_cast<int64_t>(sh) * T + t;
      if constexpr (kDtype == 1) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(y) + p * d + c * 8);
        acc[0] += bf16_lo(u.x); acc[1] += bf16_hi(u.x); acc[2] += bf16_lo(u.y); acc[3] += bf16_hi(u.y);
        acc[4] += bf16_lo(u.z); acc[5] += bf16_hi(u.z); acc[6] += bf16_lo(u.w); acc[7] += bf16_hi(u.w);
      } else {
        const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(y) + p * d + c * 8);
        const float4 a = q[0], b = q[1];
        acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
      }
    }
    if constexpr (kDtype == 1) {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(static_cast<bf16_t*>(out) + t * d + c * 8) = o;
    } else {
      float4* q = reinterpret_cast<float4*>(static_cast<float*>(out) + t * d + c * 8);
      q[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      q[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

hipError_t launch_combine(int dtype, const void* y, const int32_t* inv_perm, const float* w,
                          void* out, int64_t T, int64_t d, int k, hipStream_t s, int n_shared) {
  const int64_t n_assign = T * k;
  if (dtype == 1)
    hipLaunchKernelGGL((combine_kernel<1>), dim3(static_cast<unsigned>(T)), dim3(kCombThreads), 0, s,
                       y, inv_perm, w, out, d, k, n_assign, n_shared, T);
  else
    hipLaunchKernelGGL((combine_kernel<0>), dim3(static_cast<unsigned>(T)), dim3(kCombThreads), 0, s,
                       y, inv_perm, w, out, d, k, n_assign, n_shared, T);
  return hipGetLastError();
}

}  // namespace moe
