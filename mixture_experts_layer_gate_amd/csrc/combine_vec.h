// Device function of the weighted combine, shared by the combine kernel and the
// fused FFN kernel so that both produce the same bits:
// out[t][c..c+7] = sum_{j ascending} w[t][j] * y[inv_perm[t*k + j]][c..c+7]
// (fp32 fused multiply-add), plus y[n_assign + s*T + t] for shared experts s
// ascending, rounded once to the output type.
#pragma once
#include "common.h"

namespace moe {

template <int kDtype>
__device__ __forceinline__ void combine_vec(const void* __restrict__ y, const int32_t* __restrict__ inv_perm,
                                            const float* __restrict__ w, void* __restrict__ out, int64_t d, int k,
                                            int64_t n_assign, int n_shared, int64_t T, int64_t t, int64_t c) {
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
  // slots in groups of up to 4: the group's row loads are all issued before
  // its multiply-adds, which then run in slot order
  for (int j0 = 0; j0 < k; j0 += 4) {
    float wj[4], v[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (j0 + q < k) {
        int64_t p = inv_perm[t * k + j0 + q];
        p = p < 0 ? 0 : (p >= n_assign ? n_assign - 1 : p);
        wj[q] = w[t * k + j0 + q];
        if constexpr (kDtype == 1) {
          const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(y) + p * d + c * 8);
          v[q][0] = bf16_lo(u.x); v[q][1] = bf16_hi(u.x); v[q][2] = bf16_lo(u.y); v[q][3] = bf16_hi(u.y);
          v[q][4] = bf16_lo(u.z); v[q][5] = bf16_hi(u.z); v[q][6] = bf16_lo(u.w); v[q][7] = bf16_hi(u.w);
        } else {
          const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(y) + p * d + c * 8);
          const float4 a = src[0], b = src[1];
          v[q][0] = a.x; v[q][1] = a.y; v[q][2] = a.z; v[q][3] = a.w;
          v[q][4] = b.x; v[q][5] = b.y; v[q][6] = b.z; v[q][7] = b.w;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (j0 + q < k) {
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = __builtin_fmaf(wj[q], v[q][r], acc[r]);
      }
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

}  // namespace moe
