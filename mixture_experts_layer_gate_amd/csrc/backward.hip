// Backward pass of the MoE expert layer: everything except the grouped GEMMs
// (which are forms of the large-tile GEMM in ffn.hip; the DGrad forms read
// W1, W3 and W2 as stored, through transposing LDS loads).
//
// The pages name the backward's parts: token blocks stream through DGrad and
// WGrad, and the final top-k sum stays a step of its own (MegaFlux, section
// 2.1; section 3.2 and Figure 2). The chain rule of the forward gives, per
// assignment (t, j) of expert e with weight w and sorted row p:
//   q_p  = W2_e^T dout_t            (DGrad of FC2 before the routing weight)
//   dw   = q_p . h_p                 (= dout_t . y_p, the routing-weight gradient)
//   dh   = w q_p,  dg = dh u s (1 + g (1 - s)),  du = dh SiLU(g),  s = sigmoid(g)
//   dx_t += W1_e^T dg + W3_e^T du   (DGrad of FC1)
//   dW2_e += (w dout_t) h_p^T,  dW1_e += dg x_t^T,  dW3_e += du x_t^T   (WGrad)
// and for the softmax over the selected logits and the gate:
//   dl_j = w_j (dw_j - sum_i w_i dw_i),  dbias_e = sum dl,  dWg_e = sum dl x_t,
//   dx_t += sum_j dl_j Wg_{e_j}.
//
// Kernels here:
// * colmap_kernel: each expert's rows padded to a multiple of 64 columns in
//   the transposed activations (the WGrad K dimension), and the column -> row map;
// * gather_transpose_kernel: transposed activations for WGrad (x and dout rows
//   gathered by token, w * SiLU(g) u from g|u, dg|du), zero padding; the
//   routing weight rides on h rather than on dout, so dout enters dW2 exactly
//   and each product carries one bf16 rounding fewer;
// * swiglu_bwd_kernel: per sorted row, dg|du from q, g|u and w, and dw = q . h;
// * route_bwd_kernel: per token, the softmax backward over the k selected logits;
// * dx_combine_kernel: dx_t = sum_j (dx rows of its assignments + dl_j Wg_{e_j});
// * dwg_partial_kernel / dwg_reduce_kernel: the gate weight and bias gradients,
//   summed in a fixed order (row parts, then parts ascending).
// All reductions run in a fixed order, so results are deterministic.
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ void unpack8(const u32x4_t v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}
__device__ __forceinline__ u32x4_t pack8(const float (&f)[8]) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

// Assignment and row indices read from caller-provided arrays are clamped into
// range before they address memory (garbage in gives wrong values, never a
// stray access).
__device__ __forceinline__ int32_t clamp_assign(int32_t a, int64_t n) {
  return a < 0 ? 0 : (a >= n ? static_cast<int32_t>(n - 1) : a);
}

constexpr int kTT = 64;        // transpose tile (elements per side)
constexpr int kTP = kTT + 2;   // LDS row pitch (elements)

// One workgroup: kofs[e] = sum over e' < e of counts rounded up to 64, and
// colmap[c] = the sorted row at padded column c, or -1 for padding.
// Counts are clamped into [0, rows] and the padded offsets into [0, cols], and
// rows outside [0, rows) become padding, so inconsistent caller-provided
// counts cannot send a later kernel out of bounds.
__global__ __launch_bounds__(1024) void colmap_kernel(const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets, int E, int64_t rows,
                                                      int64_t cols, int32_t* __restrict__ kofs,
                                                      int32_t* __restrict__ colmap) {
  __shared__ int32_t ko[1025];
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int c = tid < E ? static_cast<int>((min(max(static_cast<int64_t>(counts[tid]), int64_t(0)), rows) + 63) / 64 * 64)
                        : 0;
  part[tid] = c;
  __syncthreads();
  // inclusive scan (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  if (tid == 0) ko[0] = 0;
  if (tid < E) ko[tid + 1] = static_cast<int32_t>(min(static_cast<int64_t>(part[tid]), cols));
  __syncthreads();
  if (tid == 0) kofs[0] = 0;
  if (tid < E) kofs[tid + 1] = ko[tid + 1];
  for (int64_t q = tid; q < cols; q += 1024) {
    int32_t v = -1;
    if (q < ko[E]) {
      int lo = 0, hi = E - 1;  // last e with ko[e] <= q
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (ko[mid] <= q) lo = mid; else hi = mid - 1;
      }
      const int64_t j = q - ko[lo];
      if (j < counts[lo]) {
        const int64_t pr = static_cast<int64_t>(offsets[lo]) + j;
        if (pr >= 0 && pr < rows) v = static_cast<int32_t>(pr);
      }
    }
    colmap[q] = v;
  }
}

enum GatherMode : int { kGatherTok = 0, kGatherWH = 2, kGatherDGU = 3 };

// out[i][c] for features i of one 64-wide band and padded columns c of one
// 64-wide band: the value of feature i of the row at column c (zero for padding).
//   TOK: row of src at the token of the assignment (x or dout; F = d)
//   WH:  w * SiLU(g) * u from g|u (F = f, gu rows of 2f)
//   DGU: dg|du row               (F = 2f)
template <int kG>
__global__ __launch_bounds__(256) void gather_transpose_kernel(const bf16_t* __restrict__ src,
                                                               const int32_t* __restrict__ colmap,
                                                               const int32_t* __restrict__ perm,
                                                               const float* __restrict__ topk_w, int k,
                                                               int64_t n_assign, int64_t F, int64_t src_pitch,
                                                               bf16_t* __restrict__ out, int64_t pitch) {
  __shared__ bf16_t tile[kTT * kTP];
  const int tid = threadIdx.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTT, i0 = static_cast<int64_t>(blockIdx.y) * kTT;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int cl = tid / 8 + 32 * it, f8 = (tid % 8) * 8;
    const int32_t p = colmap[c0 + cl];
    float v[8];
    if (p < 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = 0.0f;
    } else if constexpr (kG == kGatherTok) {
      const int32_t a = clamp_assign(perm[p], n_assign);
      const int64_t tok = a / k;
      unpack8(*reinterpret_cast<const u32x4_t*>(src + tok * src_pitch + i0 + f8), v);
    } else if constexpr (kG == kGatherWH) {
      const float w = topk_w[clamp_assign(perm[p], n_assign)];
      float g[8], u[8];
      unpack8(*reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(p) * src_pitch + i0 + f8), g);
      unpack8(*reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(p) * src_pitch + F + i0 + f8), u);
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = w * silu_mul(g[m], u[m]);
    } else {
      unpack8(*reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(p) * src_pitch + i0 + f8), v);
    }
    const u32x4_t pk = pack8(v);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      tile[cl * kTP + f8 + 2 * m] = static_cast<bf16_t>(pk[m] & 0xffffu);
      tile[cl * kTP + f8 + 2 * m + 1] = static_cast<bf16_t>(pk[m] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int il = tid / 8 + 32 * it, c8 = (tid % 8) * 8;
    u32x4_t v;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      v[m] = static_cast<uint32_t>(tile[(c8 + 2 * m) * kTP + il]) |
             (static_cast<uint32_t>(tile[(c8 + 2 * m + 1) * kTP + il]) << 16);
    *reinterpret_cast<u32x4_t*>(out + (i0 + il) * pitch + c0 + c8) = v;
  }
}

// Fixed-order sum over a 256-thread workgroup (wave butterflies, then the four
// wave sums in order); every thread gets the result.
__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  const float s = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return s;
}

// One workgroup per sorted row p: dh = w q, dg|du (bf16) and dw_p = q . h.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ q, const bf16_t* __restrict__ gu,
                                                         const int32_t* __restrict__ perm,
                                                         const float* __restrict__ topk_w, int64_t n_assign,
                                                         int64_t f, bf16_t* __restrict__ dgu,
                                                         float* __restrict__ dwp) {
  __shared__ float red[4];
  const int64_t p = blockIdx.x;
  const float w = topk_w[clamp_assign(perm[p], n_assign)];
  const float* qr = q + p * f;
  const bf16_t* gr = gu + p * 2 * f;
  bf16_t* dr = dgu + p * 2 * f;
  float acc = 0.0f;
  for (int64_t c = static_cast<int64_t>(threadIdx.x) * 8; c < f; c += 256 * 8) {
    float g[8], u[8], dg[8], du[8];
    unpack8(*reinterpret_cast<const u32x4_t*>(gr + c), g);
    unpack8(*reinterpret_cast<const u32x4_t*>(gr + f + c), u);
    const f32x4_t q0 = *reinterpret_cast<const f32x4_t*>(qr + c);
    const f32x4_t q1 = *reinterpret_cast<const f32x4_t*>(qr + c + 4);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float qv = m < 4 ? q0[m] : q1[m - 4];
      const float s = 1.0f / (1.0f + __expf(-g[m]));
      const float sl = g[m] * s;
      acc += qv * (sl * u[m]);
      const float dh = w * qv;
      dg[m] = dh * u[m] * (s * (1.0f + g[m] * (1.0f - s)));
      du[m] = dh * sl;
    }
    *reinterpret_cast<u32x4_t*>(dr + c) = pack8(dg);
    *reinterpret_cast<u32x4_t*>(dr + f + c) = pack8(du);
  }
  const float s = block_sum_256(acc, red);
  if (threadIdx.x == 0) dwp[p] = s;
}

// One workgroup per token: dw_j, dl_j = w_j (dw_j - sum_i w_i dw_i) (sum in slot
// order), and the optional dtopk_w [T][k] and dlogits [T][E] outputs.
__global__ __launch_bounds__(256) void route_bwd_kernel(const int32_t* __restrict__ idx,
                                                        const float* __restrict__ topk_w,
                                                        const int32_t* __restrict__ inv_perm,
                                                        const float* __restrict__ dwp, int k, int E,
                                                        int64_t n_assign, float* __restrict__ dl,
                                                        float* __restrict__ dtopk_w,
                                                        float* __restrict__ dlogits) {
  __shared__ float sdot;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t a0 = t * k;
  if (tid == 0) {
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s += topk_w[a0 + j] * dwp[clamp_assign(inv_perm[a0 + j], n_assign)];
    sdot = s;
  }
  if (dlogits)
    for (int e = tid; e < E; e += 256) dlogits[t * E + e] = 0.0f;
  __syncthreads();
  for (int j = tid; j < k; j += 256) {
    const float dw = dwp[clamp_assign(inv_perm[a0 + j], n_assign)];
    const float v = topk_w[a0 + j] * (dw - sdot);
    dl[a0 + j] = v;
    if (dtopk_w) dtopk_w[a0 + j] = dw;
    if (dlogits) dlogits[t * E + clamp_assign(idx[a0 + j], E)] = v;
  }
}

// One workgroup per token, 8 columns per thread: dx_t = sum_j (dxs[p_j] + dl_j Wg[e_j]),
// j ascending, fp32, rounded once to bf16.
__global__ __launch_bounds__(256) void dx_combine_kernel(const float* __restrict__ dxs,
                                                         const int32_t* __restrict__ inv_perm,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ dl, const bf16_t* __restrict__ wg,
                                                         int k, int E, int64_t d, bf16_t* __restrict__ dx) {
  const int64_t n_assign = static_cast<int64_t>(gridDim.x) * k;
  const int64_t t = blockIdx.x;
  for (int64_t c = static_cast<int64_t>(threadIdx.x) * 8; c < d; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int64_t a = t * k + j;
      const float* r = dxs + static_cast<int64_t>(clamp_assign(inv_perm[a], n_assign)) * d + c;
      const f32x4_t r0 = *reinterpret_cast<const f32x4_t*>(r);
      const f32x4_t r1 = *reinterpret_cast<const f32x4_t*>(r + 4);
      float gw[8];
      unpack8(*reinterpret_cast<const u32x4_t*>(wg + static_cast<int64_t>(clamp_assign(idx[a], E)) * d + c), gw);
      const float l = dl[a];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        acc[m] += m < 4 ? r0[m] : r1[m - 4];
        acc[m] += l * gw[m];
      }
    }
    *reinterpret_cast<u32x4_t*>(dx + t * d + c) = pack8(acc);
  }
}

constexpr int kGateParts = 8;  // row parts per expert in the gate-gradient sums

// grid (d / 2048 column bands, E, kGateParts): part r of expert e's sorted rows,
// part[r][e][i] = sum over its rows p (ascending) of dl_a x[token][i].
__global__ __launch_bounds__(256) void dwg_partial_kernel(const bf16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ dl, int64_t T, int k, int64_t d,
                                                          int E, float* __restrict__ part, float* __restrict__ bpart) {
  const int e = blockIdx.y, r = blockIdx.z;
  const int64_t n_assign = static_cast<int64_t>(T) * k;
  const int64_t p0 = min(max(static_cast<int64_t>(offsets[e]), int64_t(0)), n_assign);
  const int64_t n = max(min(static_cast<int64_t>(offsets[e + 1]), n_assign) - p0, int64_t(0));
  const int64_t lo = p0 + n * r / kGateParts, hi = p0 + n * (r + 1) / kGateParts;
  const int64_t c = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (c < d) {
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = 0.0f;
    // rows ascending; eight rows' loads are issued before their products are added
    constexpr int U = 8;
    int64_t p = lo;
    for (; p + U <= hi; p += U) {
      u32x4_t xr[U];
      float l[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t a = clamp_assign(perm[p + u], n_assign);
        l[u] = dl[a];
        xr[u] = *reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(a / k) * d + c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float xv[8];
        unpack8(xr[u], xv);
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] += l[u] * xv[m];
      }
    }
    for (; p < hi; ++p) {
      const int32_t a = clamp_assign(perm[p], n_assign);
      const float l = dl[a];
      float xv[8];
      unpack8(*reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(a / k) * d + c), xv);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] += l * xv[m];
    }
    float* o = part + (static_cast<int64_t>(r) * E + e) * d + c;
    *reinterpret_cast<f32x4_t*>(o) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(o + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  }
  if (blockIdx.x == 0) {
    // bias part: thread t sums rows lo + t, lo + t + 256, ... in order, then a
    // fixed-order reduction over the workgroup
    __shared__ float red[4];
    float sb = 0.0f;
    for (int64_t q = lo + threadIdx.x; q < hi; q += 256) sb += dl[clamp_assign(perm[q], n_assign)];
    sb = block_sum_256(sb, red);
    if (threadIdx.x == 0) bpart[r * E + e] = sb;
  }
}

__global__ __launch_bounds__(256) void dwg_reduce_kernel(const float* __restrict__ part,
                                                         const float* __restrict__ bpart, int64_t d, int E,
                                                         float* __restrict__ dwg, float* __restrict__ dbias) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(E) * d;
  if (i < n) {
    float s = 0.0f;
    for (int r = 0; r < kGateParts; ++r) s += part[r * n + i];
    dwg[i] = s;
  }
  if (i < E) {
    float s = 0.0f;
    for (int r = 0; r < kGateParts; ++r) s += bpart[r * E + i];
    dbias[i] = s;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.0f;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int gate_parts() { return kGateParts; }

hipError_t launch_colmap(const int32_t* counts, const int32_t* offsets, int E, int64_t rows, int64_t cols,
                         int32_t* kofs, int32_t* colmap, hipStream_t s) {
  hipLaunchKernelGGL(colmap_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, E, rows, cols, kofs, colmap);
  return hipGetLastError();
}

hipError_t launch_gather_transpose(int mode, const void* src, const int32_t* colmap, const int32_t* perm,
                                   const float* topk_w, int k, int64_t n_assign, int64_t F, int64_t src_pitch,
                                   void* out, int64_t cols, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(cols / kTT), static_cast<unsigned>(F / kTT));
  const bf16_t* sp = static_cast<const bf16_t*>(src);
  bf16_t* op = static_cast<bf16_t*>(out);
  switch (mode) {
    case 0: hipLaunchKernelGGL(gather_transpose_kernel<kGatherTok>, grid, dim3(256), 0, s, sp, colmap, perm, topk_w, k, n_assign, F, src_pitch, op, cols); break;
    case 2: hipLaunchKernelGGL(gather_transpose_kernel<kGatherWH>, grid, dim3(256), 0, s, sp, colmap, perm, topk_w, k, n_assign, F, src_pitch, op, cols); break;
    default: hipLaunchKernelGGL(gather_transpose_kernel<kGatherDGU>, grid, dim3(256), 0, s, sp, colmap, perm, topk_w, k, n_assign, F, src_pitch, op, cols); break;
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* q, const void* gu, const int32_t* perm, const float* topk_w, int64_t P,
                             int64_t f, void* dgu, float* dwp, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(static_cast<unsigned>(P)), dim3(256), 0, s, q,
                     static_cast<const bf16_t*>(gu), perm, topk_w, P, f, static_cast<bf16_t*>(dgu), dwp);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const int32_t* idx, const float* topk_w, const int32_t* inv_perm, const float* dwp,
                            int64_t T, int k, int E, float* dl, float* dtopk_w, float* dlogits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(route_bwd_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, s, idx, topk_w, inv_perm, dwp,
                     k, E, T * k, dl, dtopk_w, dlogits);
  return hipGetLastError();
}

hipError_t launch_dx_combine(const float* dxs, const int32_t* inv_perm, const int32_t* idx, const float* dl,
                             const void* wg, int64_t T, int k, int E, int64_t d, void* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(dx_combine_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, s, dxs, inv_perm, idx, dl,
                     static_cast<const bf16_t*>(wg), k, E, d, static_cast<bf16_t*>(dx));
  return hipGetLastError();
}

hipError_t launch_gate_grad(const void* x, const int32_t* perm, const int32_t* offsets, const float* dl, int64_t T,
                            int k, int64_t d, int E, float* part, float* bpart, float* dwg, float* dbias,
                            hipStream_t s) {
  hipLaunchKernelGGL(dwg_partial_kernel, dim3(static_cast<unsigned>(ceil_div(d, 2048)), E, kGateParts), dim3(256), 0,
                     s, static_cast<const bf16_t*>(x), perm, offsets, dl, T, k, d, E, part, bpart);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(dwg_reduce_kernel, dim3(static_cast<unsigned>(ceil_div(static_cast<int64_t>(E) * d, 256))),
                     dim3(256), 0, s, part, bpart, d, E, dwg, dbias);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = ceil_div(n, 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     p, n);
  return hipGetLastError();
}

}  // namespace moe
