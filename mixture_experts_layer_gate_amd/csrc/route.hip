// Router: gate logits in a fixed fp32 order, then top-k + renormalised softmax weights.
//
// The gating network scores each token against each expert and the first
// routing steps pick the top-k experts and normalise their weights
// (MegaScale-Infer, 3.2 item 2 and "Fused Kernels" steps 1 and 3).
//
// Logit order (the library's contract, so routing is reproducible bit for bit):
// lane class j = i mod 64 sums its products in increasing i starting at +0.0;
// the 64 class sums are then combined by a butterfly with offsets
// 32,16,8,4,2,1 (s_j += s_{j+off} for j < off); the bias is added last.
//
// Work mapping: a group of 64/G lanes owns a register tile of RT tokens x RE
// experts; lane q of the group owns the G consecutive lane classes
// G*q .. G*q+G-1 and loads them as one vector per row per 64-element step.
// Butterfly levels with offset >= G cross lanes of the group (lane distance
// off/G); the smaller ones stay inside a thread. Small batches use G = 1 (64
// lanes per logit) so that enough waves run; large ones use G = 8 and a
// register tile.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"
#include "route_vec.h"

namespace moe {

// A group of TPP = 64/G lanes owns a register tile of RT tokens x RE experts;
// lane q of the group owns the G consecutive lane classes G*q .. G*q+G-1.
// The K loop is unrolled by U steps of 64 elements so that U loads per row
// are in flight before the (ordered) accumulation consumes them.
template <int kDtype, int G, int RT, int RE>
__global__ __launch_bounds__(256) void gate_logits_kernel(const void* __restrict__ x,
                                                          const void* __restrict__ wg,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int T, int d,
                                                          int E, int n_eb, int64_t n_pb) {
  constexpr int TPP = 64 / G;
  constexpr int U = G == 8 ? 2 : 8;
  const int q = threadIdx.x % TPP;
  const int64_t pb = static_cast<int64_t>(blockIdx.x) * (256 / TPP) + threadIdx.x / TPP;
  const bool live = pb < n_pb;
  const int64_t pbc = live ? pb : 0;
  const int tb = static_cast<int>(pbc / n_eb), eb = static_cast<int>(pbc % n_eb);

  int64_t xrow[RT], wrow[RE];
#pragma unroll
  for (int r = 0; r < RT; ++r) xrow[r] = static_cast<int64_t>(min(tb * RT + r, T - 1)) * d;
#pragma unroll
  for (int r = 0; r < RE; ++r) wrow[r] = static_cast<int64_t>(min(eb * RE + r, E - 1)) * d;

  float acc[RT][RE][G];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b)
#pragma unroll
      for (int r = 0; r < G; ++r) acc[a][b][r] = 0.0f;

  int i0 = q * G;
  // full batches of U steps: all loads first, then the FMAs in order
  for (; i0 + (U - 1) * 64 < d; i0 += U * 64) {
    float xv[U][RT][G], wv[U][RE][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int a = 0; a < RT; ++a) loadG<kDtype, G>(x, xrow[a] + i0 + u * 64, xv[u][a]);
#pragma unroll
      for (int b = 0; b < RE; ++b) loadG<kDtype, G>(wg, wrow[b] + i0 + u * 64, wv[u][b]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b = 0; b < RE; ++b)
#pragma unroll
          for (int r = 0; r < G; ++r) acc[a][b][r] = mac<kDtype>(xv[u][a][r], wv[u][b][r], acc[a][b][r]);
  }
  for (; i0 < d; i0 += 64) {
    float xv[RT][G], wv[RE][G];
#pragma unroll
    for (int a = 0; a < RT; ++a) loadG<kDtype, G>(x, xrow[a] + i0, xv[a]);
#pragma unroll
    for (int b = 0; b < RE; ++b) loadG<kDtype, G>(wg, wrow[b] + i0, wv[b]);
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
      for (int b = 0; b < RE; ++b)
#pragma unroll
        for (int r = 0; r < G; ++r) acc[a][b][r] = mac<kDtype>(xv[a][r], wv[b][r], acc[a][b][r]);
  }

  // Butterfly over class j = G*q + r: offsets >= G pair lane q with q + off/G,
  // smaller offsets stay inside the thread.
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b) {
#pragma unroll
      for (int off = 32; off >= G; off >>= 1)
#pragma unroll
        for (int r = 0; r < G; ++r) acc[a][b][r] = acc[a][b][r] + __shfl_down(acc[a][b][r], off / G, TPP);
#pragma unroll
      for (int off = G / 2; off >= 1; off >>= 1)
#pragma unroll
        for (int r = 0; r < off; ++r) acc[a][b][r] = acc[a][b][r] + acc[a][b][r + off];
    }
  if (!live || q != 0) return;
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b) {
      const int t = tb * RT + a, e = eb * RE + b;
      if (t < T && e < E) {
        const float bv = bias ? bias[e] : 0.0f;
        logits[static_cast<int64_t>(t) * E + e] = acc[a][b][0] + bv;
      }
    }
}

template <int kDtype, int G, int RT, int RE>
static hipError_t gate_launch(const void* x, const void* wg, const float* bias, float* logits,
                              int64_t T, int64_t d, int E, hipStream_t s) {
  constexpr int TPP = 64 / G;
  const int n_tb = static_cast<int>((T + RT - 1) / RT);
  const int n_eb = (E + RE - 1) / RE;
  const int64_t n_pb = static_cast<int64_t>(n_tb) * n_eb;
  const int64_t per_block = 256 / TPP;
  const int64_t blocks = (n_pb + per_block - 1) / per_block;
  hipLaunchKernelGGL((gate_logits_kernel<kDtype, G, RT, RE>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, x, wg, bias, logits, static_cast<int>(T), static_cast<int>(d),
                     E, n_eb, n_pb);
  return hipGetLastError();
}

// LDS-staged variant for bf16 gates with many experts (d % 64 == 0). A
// workgroup owns 16 tokens x 32 experts; K is walked in chunks of 128 that
// are loaded as bf16, converted to fp32 once and stored in LDS (two
// buffers), so the inner loop is LDS reads and FMAs only. Lane mapping and
// summation order are those of gate_logits_kernel with G = 4, RT = 4, RE = 8:
// 16 lane groups of 16 lanes, group (tg, eg) = tokens 4tg..4tg+3 x experts
// 8eg..8eg+7, lane q holding classes 4q..4q+3, each class summed in
// increasing element order, then the same butterfly and bias add.
constexpr int kLdsTT = 16, kLdsTE = 32, kLdsKC = 128;

// G classes per lane (lane q of a group of 64 / G lanes holds classes Gq ..
// Gq + G - 1), RT tokens x RE experts per group; (G, RT, RE) = (4, 4, 8) or
// (2, 8, 8): the same 16 x 32 workgroup tile, the same contract order. The
// second reads a third fewer LDS bytes per FMA but measured 10 % slower on
// the 4096 x 7168 x 256 gate (more, narrower reads); it is selected only by
// MOE_GATE_CFG=lds2.
template <int G, int RT, int RE>
__global__ __launch_bounds__(256, 2) void gate_lds_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                                       const float* __restrict__ bias, float* __restrict__ logits,
                                                       int T, int d, int E) {
  constexpr int TPP = 64 / G, NEG = kLdsTE / RE;  // lanes per group, expert groups per tile
  static_assert((256 / TPP) * RT * RE == kLdsTT * kLdsTE, "the groups cover the workgroup tile");
  typedef float fvec_t __attribute__((ext_vector_type(G)));
  constexpr int XS = kLdsTT * kLdsKC, WS = kLdsTE * kLdsKC;  // floats per buffer
  __shared__ __attribute__((aligned(16))) float lx[2][XS];
  __shared__ __attribute__((aligned(16))) float lw[2][WS];
  const int tid = threadIdx.x, q = tid % TPP, grp = tid / TPP;
  const int tg = grp / NEG, eg = grp % NEG;
  const int t0 = blockIdx.y * kLdsTT, e0 = blockIdx.x * kLdsTE;

  // staging: 16-byte (8-element) pieces; x tile 16 x 128 = 256 pieces (one
  // per thread), w tile 32 x 128 = 512 pieces (two per thread)
  const int xr = tid / 16, xc = (tid % 16) * 8;
  const bf16_t* xsrc = x + static_cast<int64_t>(min(t0 + xr, T - 1)) * d + xc;
  const bf16_t* wsrc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) wsrc[h] = wg + static_cast<int64_t>(min(e0 + xr + 16 * h, E - 1)) * d + xc;
  u32x4_t rx, rw[2];
  const int nch = (d + kLdsKC - 1) / kLdsKC;
  auto gload = [&](int c) {  // chunk c, clamped to the row: a short last chunk reads valid memory, never used
    const int k0 = min(c * kLdsKC, d - kLdsKC < 0 ? 0 : d - kLdsKC);
    const int off = c * kLdsKC + xc < d ? c * kLdsKC : k0;
    rx = *reinterpret_cast<const u32x4_t*>(xsrc + off);
#pragma unroll
    for (int h = 0; h < 2; ++h) rw[h] = *reinterpret_cast<const u32x4_t*>(wsrc[h] + off);
  };
  auto lstore = [&](int b) {
    float* px = &lx[b][xr * kLdsKC + xc];
    reinterpret_cast<f32x4_t*>(px)[0] = f32x4_t{bf16_lo(rx[0]), bf16_hi(rx[0]), bf16_lo(rx[1]), bf16_hi(rx[1])};
    reinterpret_cast<f32x4_t*>(px)[1] = f32x4_t{bf16_lo(rx[2]), bf16_hi(rx[2]), bf16_lo(rx[3]), bf16_hi(rx[3])};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float* pw = &lw[b][(xr + 16 * h) * kLdsKC + xc];
      reinterpret_cast<f32x4_t*>(pw)[0] =
          f32x4_t{bf16_lo(rw[h][0]), bf16_hi(rw[h][0]), bf16_lo(rw[h][1]), bf16_hi(rw[h][1])};
      reinterpret_cast<f32x4_t*>(pw)[1] =
          f32x4_t{bf16_lo(rw[h][2]), bf16_hi(rw[h][2]), bf16_lo(rw[h][3]), bf16_hi(rw[h][3])};
    }
  };

  float acc[RT][RE][G];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b)
#pragma unroll
      for (int r = 0; r < G; ++r) acc[a][b][r] = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int b = c & 1;
    if (c + 1 < nch) gload(c + 1);
    const int steps = min(kLdsKC, d - c * kLdsKC) / 64;  // d % 64 == 0
#pragma unroll 1
    for (int st = 0; st < steps; ++st) {
      fvec_t xv[RT], wv[RE];
#pragma unroll
      for (int a = 0; a < RT; ++a) xv[a] = *reinterpret_cast<const fvec_t*>(&lx[b][(RT * tg + a) * kLdsKC + st * 64 + G * q]);
#pragma unroll
      for (int e = 0; e < RE; ++e) wv[e] = *reinterpret_cast<const fvec_t*>(&lw[b][(RE * eg + e) * kLdsKC + st * 64 + G * q]);
#pragma unroll
      for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int e = 0; e < RE; ++e)
#pragma unroll
          for (int r = 0; r < G; ++r) acc[a][e][r] = __builtin_fmaf(xv[a][r], wv[e][r], acc[a][e][r]);
    }
    if (c + 1 < nch) lstore(b ^ 1);  // buffer b^1 was last read in step c-1, before the barrier below it
    __syncthreads();
  }

  // The butterfly over the 64 class sums, in-lane: for each of the lane's RT
  // token rows in turn, every lane writes its G class sums of its RE logits
  // to LDS, and one thread per logit reads back all 64 and adds the same pairs
  // in the same order (s_j += s_{j+off}, off = 32 .. 1), then the bias. Row L
  // of the [logits][64] block holds 4-class chunk k at slot k ^ (L % 16), so
  // 16 threads reading chunk k of 16 consecutive rows hit 16 distinct banks.
  constexpr int NL = (256 / TPP) * RE;  // logits per token row of the lanes
  static_assert(NL * 64 <= 2 * WS, "a token row's class sums fit in the weight buffers");
  float* red = &lw[0][0];
  auto slot_of = [](int L, int cls) { return L * 64 + ((cls & ~3) ^ (4 * (L % 16))) + (cls & 3); };
#pragma unroll
  for (int a = 0; a < RT; ++a) {
#pragma unroll
    for (int e = 0; e < RE; ++e) {
      const int L = grp * RE + e;
      *reinterpret_cast<fvec_t*>(&red[slot_of(L, G * q)]) = *reinterpret_cast<const fvec_t*>(&acc[a][e][0]);
    }
    __syncthreads();
    if (tid < NL) {
      const int L = tid;
      float sv[64];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&red[slot_of(L, 4 * k)]);
        sv[4 * k] = v[0];
        sv[4 * k + 1] = v[1];
        sv[4 * k + 2] = v[2];
        sv[4 * k + 3] = v[3];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int j = 0; j < off; ++j) sv[j] = sv[j] + sv[j + off];
      const int lg = L / RE, le = L % RE;
      const int t = t0 + RT * (lg / NEG) + a, ex = e0 + RE * (lg % NEG) + le;
      if (t < T && ex < E) logits[static_cast<int64_t>(t) * E + ex] = sv[0] + (bias ? bias[ex] : 0.0f);
    }
    __syncthreads();  // the block is read out before the next token row overwrites it
  }
}

template <int G, int RT, int RE>
static hipError_t gate_lds_launch(const void* x, const void* wg, const float* bias, float* logits, int64_t T,
                                  int64_t d, int E, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((E + kLdsTE - 1) / kLdsTE), static_cast<unsigned>((T + kLdsTT - 1) / kLdsTT));
  hipLaunchKernelGGL((gate_lds_kernel<G, RT, RE>), grid, dim3(256), 0, s, static_cast<const bf16_t*>(x),
                     static_cast<const bf16_t*>(wg), bias, logits, static_cast<int>(T), static_cast<int>(d), E);
  return hipGetLastError();
}

// Gate logits on the fp32 matrix cores, in the contract order. An fp32 MFMA
// with K = 1 (v_mfma_f32_32x32x1f32: two 32 x 32 outer-product blocks) adds
// one exact product to each output and rounds once, which is exactly fmaf;
// a class chain of such MFMAs, one per element of the class in increasing
// order from +0.0, therefore gives the bits of the VALU chains, at twice the
// VALU rate (256 fp32 FLOP per clock and CU) and with one 16-byte LDS read
// per row per K step instead of one per lane class group.
// A workgroup of 8 waves owns 32 tokens x 32 experts; wave w owns the lane
// classes 8w .. 8w + 7, its MFMA i of a 64-element step covering classes
// 8w + 2i (block 0) and 8w + 2i + 1 (block 1); lane l feeds block l / 32 with
// token row (A) and expert row (B) l % 32, both read as the 8 bf16 elements
// 8w .. 8w + 7 of the step, of which it takes the even (block 0) or odd ones
// (one byte permute each turns them into fp32). x and Wg stream through LDS
// as bf16 in chunks of kMfKC elements (rows padded by 16 bytes, so the 16 rows
// of a read pass fall in distinct banks), double-buffered; each wave reads a
// step's operands one step ahead of its MFMAs. The class sums of every logit
// are then finished as in gate_lds_kernel: written to LDS, 8 token rows at a
// time, and added by one thread per logit in the butterfly's order, then the
// bias. DeepSeek-V3-shaped gate (4096 tokens x 7168 x 256 experts): 0.21 ms
// against 0.33-0.35 ms for gate_lds_kernel.
constexpr int kMfT = 32, kMfE = 32, kMfKC = 512;
constexpr int kMfRow = kMfKC * 2 + 16;     // bytes per staged row
constexpr int kMfTile = (kMfT + kMfE) * kMfRow;  // bytes per buffer (x rows, then Wg rows)
constexpr int kMfPieces = (kMfT + kMfE) * (kMfKC / 8) / 512;  // 16-byte pieces per thread per chunk
static_assert(2 * kMfTile >= 8 * kMfE * 64 * 4, "a round of 8 token rows' class sums fits in the buffers");

__global__ __launch_bounds__(512) void gate_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                                        const float* __restrict__ bias, float* __restrict__ logits,
                                                        int T, int d, int E) {
  typedef float f32x32_t __attribute__((ext_vector_type(32)));
  __shared__ __attribute__((aligned(16))) char lds[2 * kMfTile];
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, half = l / 32, row = l % 32;
  const int t0 = blockIdx.y * kMfT, e0 = blockIdx.x * kMfE;

  // staging: piece p (16 bytes) = row p / (kMfKC / 8) of the 64 tile rows (x
  // rows first), column piece p % (kMfKC / 8); rows past T or E repeat the
  // last row, and pieces past d re-read the row's last piece (never used)
  constexpr int PPR = kMfKC / 8;
  const bf16_t* src[kMfPieces];
  int dst[kMfPieces], pcol[kMfPieces];
#pragma unroll
  for (int i = 0; i < kMfPieces; ++i) {
    const int p = tid + 512 * i, r = p / PPR, pc = p % PPR;
    src[i] = r < kMfT ? x + static_cast<int64_t>(min(t0 + r, T - 1)) * d
                      : wg + static_cast<int64_t>(min(e0 + r - kMfT, E - 1)) * d;
    dst[i] = r * kMfRow + pc * 16;
    pcol[i] = pc * 8;
  }
  u32x4_t stage[kMfPieces];
  auto gload = [&](int c) {
#pragma unroll
    for (int i = 0; i < kMfPieces; ++i) {
      const int col = min(c * kMfKC + pcol[i], d - 8);
      stage[i] = *reinterpret_cast<const u32x4_t*>(src[i] + col);
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < kMfPieces; ++i) *reinterpret_cast<u32x4_t*>(lds + b * kMfTile + dst[i]) = stage[i];
  };

  f32x32_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 32; ++r) acc[i][r] = 0.0f;

  const int nch = (d + kMfKC - 1) / kMfKC;
  // block 0 takes the even (low) halves, block 1 the odd (high) ones: byte
  // selectors of v_perm_b32 over the word in both sources (0..3: its bytes;
  // 12: a zero byte)
  const uint32_t sel = half ? 0x03020c0cu : 0x01000c0cu;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int b = c & 1;
    if (c + 1 < nch) gload(c + 1);
    const int steps = min(kMfKC, d - c * kMfKC) / 64;  // d % 64 == 0
    const char* xrow = lds + b * kMfTile + row * kMfRow + w * 16;
    const char* wrow = xrow + kMfT * kMfRow;
    // the next step's operands are read before this step's MFMAs are issued
    // (two register sets; a read past the chunk's last step re-reads it, unused)
    auto mma = [&](const u32x4_t& xa, const u32x4_t& wb) {
      // bf16 -> fp32 by one byte permute per operand (the half's two bytes to
      // the top, zeros below), all eight before the four MFMAs
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = __uint_as_float(__builtin_amdgcn_perm(xa[i], xa[i], sel));
        bv[i] = __uint_as_float(__builtin_amdgcn_perm(wb[i], wb[i], sel));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x1f32(av[i], bv[i], acc[i], 0, 0, 0);
    };
    u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(xrow), w0 = *reinterpret_cast<const u32x4_t*>(wrow);
#pragma unroll 1
    for (int st = 0; st < steps; st += 2) {
      const int n1 = min(st + 1, steps - 1) * 128, n2 = min(st + 2, steps - 1) * 128;
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(xrow + n1), w1 = *reinterpret_cast<const u32x4_t*>(wrow + n1);
      __builtin_amdgcn_sched_barrier(0);
      mma(x0, w0);
      __builtin_amdgcn_sched_barrier(0);
      x0 = *reinterpret_cast<const u32x4_t*>(xrow + n2);
      w0 = *reinterpret_cast<const u32x4_t*>(wrow + n2);
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < steps) mma(x1, w1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c + 1 < nch) lstore(b ^ 1);  // buffer b^1 was last read in chunk c-1, before the barrier below it
    __syncthreads();
  }

  // Finish: accumulator register k (of a block's 16) of lane l holds token
  // row 8(k/4) + 4(l/32) + k%4 and expert column l%32, so round q (token rows
  // 8q .. 8q+7) takes registers 4q .. 4q+3. Logit (m, n) of the round keeps
  // its 64 class sums at [p = m*32 + n][64], 4-class chunk k at slot
  // k ^ (p % 16) (16 consecutive logits in 16 distinct bank groups).
  float* red = reinterpret_cast<float*>(lds);
  auto slot = [](int p, int chunk) { return p * 64 + ((chunk ^ (p % 16)) * 4); };
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int k = 4 * q + kk;
      const int p = (4 * half + kk) * 32 + row;
      // classes 8w .. 8w+3 and 8w+4 .. 8w+7: (MFMA i, block) = (0,0) (0,1) (1,0) (1,1), then (2,*) (3,*)
      *reinterpret_cast<f32x4_t*>(&red[slot(p, 2 * w)]) = f32x4_t{acc[0][k], acc[0][16 + k], acc[1][k], acc[1][16 + k]};
      *reinterpret_cast<f32x4_t*>(&red[slot(p, 2 * w + 1)]) =
          f32x4_t{acc[2][k], acc[2][16 + k], acc[3][k], acc[3][16 + k]};
    }
    __syncthreads();
    if (tid < 8 * kMfE) {
      const int p = tid;
      float sv[64];
#pragma unroll
      for (int ch = 0; ch < 16; ++ch) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&red[slot(p, ch)]);
        sv[4 * ch] = v[0];
        sv[4 * ch + 1] = v[1];
        sv[4 * ch + 2] = v[2];
        sv[4 * ch + 3] = v[3];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int j = 0; j < off; ++j) sv[j] = sv[j] + sv[j + off];
      const int t = t0 + 8 * q + p / 32, ex = e0 + p % 32;
      if (t < T && ex < E) logits[static_cast<int64_t>(t) * E + ex] = sv[0] + (bias ? bias[ex] : 0.0f);
    }
    __syncthreads();  // the block is read out before the next round overwrites it
  }
}

static hipError_t gate_mfma_launch(const void* x, const void* wg, const float* bias, float* logits, int64_t T,
                                   int64_t d, int E, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((E + kMfE - 1) / kMfE), static_cast<unsigned>((T + kMfT - 1) / kMfT));
  hipLaunchKernelGGL(gate_mfma_kernel, grid, dim3(512), 0, s, static_cast<const bf16_t*>(x),
                     static_cast<const bf16_t*>(wg), bias, logits, static_cast<int>(T), static_cast<int>(d), E);
  return hipGetLastError();
}

// Whether the gate of a T x d x E batch runs on gate_mfma_kernel: bf16, d a
// multiple of 64, at least 32 experts and at least one 32 x 32 workgroup tile
// per CU's worth (256); MOE_GATE_CFG=mfma forces it where the kernel can run,
// any other valid setting forces a VALU tile.
static bool mfma_gate_ok(int dtype, int64_t T, int64_t d) {
  return dtype == 1 && d % 64 == 0 && T <= 65535 * static_cast<int64_t>(kMfT);
}
bool gate_uses_mfma(int dtype, int64_t T, int64_t d, int E) {
  if (!mfma_gate_ok(dtype, T, d)) return false;
  if (const char* env = getenv("MOE_GATE_CFG")) {
    if (strcmp(env, "mfma") == 0) return true;
    int g = 0, rt = 0, re = 0;
    if (strcmp(env, "lds") == 0 || strcmp(env, "lds2") == 0 || sscanf(env, "%d,%d,%d", &g, &rt, &re) == 3) return false;
  }
  return E >= kMfE && ((T + kMfT - 1) / kMfT) * ((E + kMfE - 1) / kMfE) >= 256;
}

template <int kDtype>
static hipError_t gate_dispatch(const void* x, const void* wg, const float* bias, float* logits,
                                int64_t T, int64_t d, int E, hipStream_t s) {
  // Most work per thread (big register tile, few conversions per FMA) that
  // still gives >= 2048 waves (8 per CU); otherwise the narrowest mapping.
  // On the 4096 x 7168 x 256 gate, tiles of 2 classes x 4 tokens x 8 experts
  // measured fastest; tiles that force one wave per SIMD were slower.
  auto waves = [&](int g, int rt, int re) {
    const int64_t pbs = ((T + rt - 1) / rt) * ((E + re - 1) / re);
    return pbs * (64 / g) / kWave;
  };
  const int64_t want = 2048;
  const bool lds_ok = kDtype == 1 && d % 64 == 0 && d >= kLdsKC && T <= 65535 * static_cast<int64_t>(kLdsTT);
  if (const char* env = getenv("MOE_GATE_CFG")) {  // tuning: "lds" or "G,RT,RE" among the instantiated tiles
    if (lds_ok && strcmp(env, "lds") == 0) return gate_lds_launch<4, 4, 8>(x, wg, bias, logits, T, d, E, s);
    if (lds_ok && strcmp(env, "lds2") == 0) return gate_lds_launch<2, 8, 8>(x, wg, bias, logits, T, d, E, s);
    int g = 0, rt = 0, re = 0;
    if (sscanf(env, "%d,%d,%d", &g, &rt, &re) == 3) {
      if (g == 4 && rt == 4 && re == 4) return gate_launch<kDtype, 4, 4, 4>(x, wg, bias, logits, T, d, E, s);
      if (g == 2 && rt == 4 && re == 8) return gate_launch<kDtype, 2, 4, 8>(x, wg, bias, logits, T, d, E, s);
      if (g == 8 && rt == 2 && re == 4) return gate_launch<kDtype, 8, 2, 4>(x, wg, bias, logits, T, d, E, s);
    }
  }
  // many experts and tokens: the matrix-core tile (32 tokens x 32 experts per
  // workgroup), else the LDS-staged VALU tile (16 x 32)
  if (gate_uses_mfma(kDtype, T, d, E)) return gate_mfma_launch(x, wg, bias, logits, T, d, E, s);
  if (lds_ok && E >= kLdsTE && ((T + kLdsTT - 1) / kLdsTT) * ((E + kLdsTE - 1) / kLdsTE) >= 1024)
    return gate_lds_launch<4, 4, 8>(x, wg, bias, logits, T, d, E, s);
  if (E >= 8 && waves(2, 4, 8) >= want) return gate_launch<kDtype, 2, 4, 8>(x, wg, bias, logits, T, d, E, s);
  if (E >= 4 && waves(8, 2, 4) >= want) return gate_launch<kDtype, 8, 2, 4>(x, wg, bias, logits, T, d, E, s);
  if (E >= 2 && waves(8, 2, 2) >= want) return gate_launch<kDtype, 8, 2, 2>(x, wg, bias, logits, T, d, E, s);
  if (E >= 2 && waves(8, 1, 2) >= want) return gate_launch<kDtype, 8, 1, 2>(x, wg, bias, logits, T, d, E, s);
  if (waves(8, 1, 1) >= want) return gate_launch<kDtype, 8, 1, 1>(x, wg, bias, logits, T, d, E, s);
  if (waves(4, 1, 1) >= want) return gate_launch<kDtype, 4, 1, 1>(x, wg, bias, logits, T, d, E, s);
  if (waves(2, 1, 1) >= want) return gate_launch<kDtype, 2, 1, 1>(x, wg, bias, logits, T, d, E, s);
  return gate_launch<kDtype, 1, 1, 1>(x, wg, bias, logits, T, d, E, s);
}

hipError_t launch_gate_logits(int dtype, const void* x, const void* wg, const float* bias,
                              float* logits, int64_t T, int64_t d, int E, hipStream_t s) {
  if (dtype == 1) return gate_dispatch<1>(x, wg, bias, logits, T, d, E, s);
  return gate_dispatch<0>(x, wg, bias, logits, T, d, E, s);
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token. Order: logit descending, equal logits to the
// lower expert index (IEEE compare, so -0 == +0). Weights: softmax over the k
// selected logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  __shared__ float sel_v[4][kMaxE];
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  topk_row(logits + static_cast<int64_t>(t) * E, E, k, idx + static_cast<int64_t>(t) * k,
           w + static_cast<int64_t>(t) * k, sel_v[wv]);
}

// Gate and top-k of small batches in one launch: workgroup t holds token t,
// wave e computes logit (t, e) in the contract order (lane q sums class q,
// elements q, q + 64, .. in order, then the butterfly over offsets 32 .. 1 and
// the bias: gate_logits_kernel's order with one class per lane), and wave 0
// then selects the token's top k from the logits in LDS.
template <int kDtype>
__global__ __launch_bounds__(1024) void route_small_kernel(const void* __restrict__ x, const void* __restrict__ wg,
                                                           const float* __restrict__ bias, float* __restrict__ logits,
                                                           int T, int d, int E, int k, int32_t* __restrict__ idx,
                                                           float* __restrict__ w) {
  __shared__ float srow[kRouteSmallMaxE];
  __shared__ float sel[kMaxE];
  const int lane = threadIdx.x & 63, e = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const float l = gate_logit_wave<kDtype>(x, wg, bias, t, e, d);
  if (lane == 0) {
    srow[e] = l;
    logits[static_cast<int64_t>(t) * E + e] = l;
  }
  __syncthreads();
  if (e == 0)
    topk_row(srow, E, k, idx + static_cast<int64_t>(t) * k, w + static_cast<int64_t>(t) * k, sel);
}

bool route_small_ok(int64_t T, int E) {
  if (getenv("MOE_GATE_CFG")) return false;  // a forced gate tiling keeps the separate launches
  return T >= 1 && E <= kRouteSmallMaxE && T * E <= 4096;
}

hipError_t launch_route_small(int dtype, const void* x, const void* wg, const float* bias, float* logits, int64_t T,
                              int64_t d, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(route_small_kernel<1>, dim3(static_cast<unsigned>(T)), dim3(64 * E), 0, s, x, wg, bias, logits,
                       static_cast<int>(T), static_cast<int>(d), E, k, idx, w);
  else
    hipLaunchKernelGGL(route_small_kernel<0>, dim3(static_cast<unsigned>(T)), dim3(64 * E), 0, s, x, wg, bias, logits,
                       static_cast<int>(T), static_cast<int>(d), E, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                       hipStream_t s) {
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, logits,
                     static_cast<int>(T), E, k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
