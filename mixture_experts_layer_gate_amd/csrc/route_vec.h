// Device functions of the router shared by the gate and top-k kernels and the
// fused layer launch, so that all of them produce the same bits: element loads
// as fp32, the multiply-add of the fixed logit order, one logit per wave in that
// order, and the wave top-k with its renormalised softmax weights.
//
// Logit order (the library's contract, so routing is reproducible bit for bit):
// lane class j = i mod 64 sums its products in increasing i starting at +0.0;
// the 64 class sums are then combined by a butterfly with offsets
// 32,16,8,4,2,1 (s_j += s_{j+off} for j < off); the bias is added last.
#pragma once
#include "common.h"

namespace moe {

// G consecutive elements as fp32 (G = 1, 2, 4 or 8; 2*G bytes for bf16, 4*G for fp32).
template <int kDtype, int G>
__device__ __forceinline__ void loadG(const void* base, int64_t elem_off, float (&v)[G]) {
  if constexpr (kDtype == 1) {
    const bf16_t* p = static_cast<const bf16_t*>(base) + elem_off;
    if constexpr (G == 8) {
      const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(u[i]); v[2 * i + 1] = bf16_hi(u[i]); }
    } else if constexpr (G == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    } else if constexpr (G == 2) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      v[0] = bf16_lo(u); v[1] = bf16_hi(u);
    } else {
      v[0] = __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
  } else {
    const float* p = static_cast<const float*>(base) + elem_off;
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = p[i];
  }
}

// acc + x*w with the product rounded first. For bf16 operands the product is
// exact in fp32, so a fused multiply-add gives the same bits; fp32 operands
// need the separate multiply.
template <int kDtype>
__device__ __forceinline__ float mac(float x, float w, float acc) {
  if constexpr (kDtype == 1) {
    return __builtin_fmaf(x, w, acc);
  } else {
#pragma clang fp contract(off)
    const float p = x * w;
    return acc + p;
  }
}

// Logit (t, e) computed by one wave in the contract order: lane q sums class q
// (elements q, q + 64, .. in order), then the butterfly over offsets 32 .. 1
// and the bias. Every lane calls it; lane 0 holds the logit. The loads of U
// elements per lane are issued before their multiply-adds: a logit of a
// small batch is a chain of d / (64 U) memory round trips.
template <int kDtype, int U = 32>
__device__ __forceinline__ float gate_logit_wave(const void* __restrict__ x, const void* __restrict__ wg,
                                                 const float* __restrict__ bias, int64_t t, int e, int64_t d) {
  const int lane = threadIdx.x & 63;
  const int64_t xrow = t * d, wrow = static_cast<int64_t>(e) * d;
  float acc = 0.0f;
  int64_t i0 = lane;
  for (; i0 + (U - 1) * 64 < d; i0 += U * 64) {
    float xv[U][1], wv[U][1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      loadG<kDtype, 1>(x, xrow + i0 + u * 64, xv[u]);
      loadG<kDtype, 1>(wg, wrow + i0 + u * 64, wv[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = mac<kDtype>(xv[u][0], wv[u][0], acc);
  }
  for (; i0 < d; i0 += 64) {
    float xv[1], wv[1];
    loadG<kDtype, 1>(x, xrow + i0, xv);
    loadG<kDtype, 1>(wg, wrow + i0, wv);
    acc = mac<kDtype>(xv[0], wv[0], acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_down(acc, off, 64);
  return acc + (bias ? bias[e] : 0.0f);
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token. Order: logit descending, equal logits to the
// lower expert index (IEEE compare, so -0 == +0). Weights: softmax over the k
// selected logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
constexpr int kMaxE = 1024;
constexpr int kRouteSmallMaxE = 16;  // experts of the one-launch gate + top-k (one wave each)
constexpr int kPerLane = kMaxE / kWave;

__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

// Top-k of one token's E logits by one wave (every lane calls it): k rounds
// of a wave arg-max, then the weights. sel: kMaxE floats of this wave's LDS.
__device__ __forceinline__ void topk_row(const float* row, int E, int k, int32_t* __restrict__ idx_row,
                                         float* __restrict__ w_row, float* sel) {
  const int lane = threadIdx.x & 63;
  float v[kPerLane];
  bool taken[kPerLane];
  const int per = (E + kWave - 1) / kWave;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + i * kWave;
    const bool ok = i < per && e < E;
    v[i] = ok ? row[e] : 0.0f;
    taken[i] = !ok;
  }
  float v0 = 0.0f, sum = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + i * kWave;
      if (!taken[i] && (be == 0x7fffffff || better(v[i], e, bv, be))) { bv = v[i]; be = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (oe != 0x7fffffff && (be == 0x7fffffff || better(ov, oe, bv, be))) { bv = ov; be = oe; }
    }
    // every lane now holds the same winner (bv, be)
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      if (lane + i * kWave == be) taken[i] = true;
    if (j == 0) v0 = bv;
    sum += expf(bv - v0);
    if (lane == 0) {
      idx_row[j] = be;
      sel[j] = bv;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float inv = 1.0f / sum;
  for (int j = lane; j < k; j += kWave) w_row[j] = expf(sel[j] - v0) * inv;
}

}  // namespace moe
