// Grouped SwiGLU expert FFN: FC1 (gate and up projections, SiLU * mul fused in
// the epilogue) and FC2 (down projection), over tile-aligned m-blocks.
//
// Expert definition: three matrices per expert, gate and up of size d x f and
// down of size f x d (Piper, section III-A); FC1 then FC2 tiles per expert
// (MegaFlux, section 2.1); token blocks of at most 128 rows, one partial block
// per expert at most (MegaFlux, section 3.1).
//
// Kernel shape: 256 threads (4 waves as 2 x 2), tile of 128 rows x 128 weight
// rows, K step 64, bf16 MFMA 32x32x16 (fp32 data: 32x32x2). Each wave owns 64
// rows x 2 column blocks of 32. FC1 pairs the column blocks as (gate, up) of
// the same 32 output columns, so SiLU(g) * u is formed in registers. A rows
// are gathered through perm (FC1) or read contiguously (FC2). Tiles are taken
// from a persistent loop over (n-block, m-block) pairs; waves whose 32-row
// sub-blocks lie entirely past the block's rows skip their MFMAs.
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <utility>

#include "combine_vec.h"
#include "common.h"
#include "dispatch_block.h"
#include "kernels.h"
#include "route_vec.h"

namespace moe {

constexpr int kBM = 128;     // rows per tile (== kBlockRows)
constexpr int kBNW = 128;    // weight rows per tile
constexpr int kBK = 64;      // K per step
constexpr int kThreads = 256;
static_assert(kBM == kBlockRows, "small-tile rows must match the plan's smallest block rows");

struct GemmArgs {
  const void* A;          // FC1: x [T][K]; FC2: h [rows][K]
  const int32_t* perm;    // FC1: sorted row -> assignment (routed rows)
  int ktop;               // FC1: token = perm[p] / ktop
  int64_t T;              // FC1: token count (clamp; shared rows: token = (p - n_routed) % T)
  const void* B0;         // FC1: W1 [E][N][K]; FC2: W2 [E][N][K]
  const void* B1;         // FC1: W3 [E][N][K]
  void* C;                // FC1: h [rows][N]; FC2: y [rows][N]
  const int4* mblocks;    // (expert, first sorted row, rows, tile group)
  const int32_t* n_mblocks;
  int64_t K, N;
  int64_t n_routed;       // sorted rows covered by perm; rows after them belong to shared experts
  const void* S0;         // shared experts' W1 (FC1) or W2 (FC2), [S][N][K]
  const void* S1;         // shared experts' W3 (FC1)
  int E_routed;           // experts e >= E_routed are shared expert e - E_routed
  // g | u form: h [rows][N] bf16 (from the fp32 sums) as well when non-null. Weight gradients
  // (C[e] = A_e B_e^T with K = the expert's padded rows): the second output
  // tensor, for output rows >= split.
  void* C2;
  const int32_t* kofs;    // [E+1] first padded column of each expert in A and B
  int64_t pitch;          // row pitch (elements) of the transposed operands A and B
  int64_t M;              // output rows per expert (rows of A)
  int64_t split;          // output rows per output tensor (M, or M / 2 with C2)
  int n_experts;
  // rows of the m-block's A (non-gathered forms): row pitch in elements (0 = K)
  // and first column; fp32 forms: add to C instead of storing
  int64_t a_pitch, a_col0;
  int accumulate;
  int out_bf16;           // weight gradients: store C (and C2) as bf16, rounded to nearest even
  // split K: the tiles past the last full round of split_target workgroups
  // (all of them in a launch with fewer tiles than CUs) have their K steps
  // cut into parts, each part's fp32 accumulators go to `partial`
  // ([part slot][BM][BN]), and splitk_reduce_kernel sums them in part order.
  // At most `splits` parts, at most split_target part slots (one round of the
  // persistent grid), at most partial_cap of them stored; after full rounds,
  // at least tail_min parts (2 if unset), else no split.
  float* partial;
  int splits, split_target, partial_cap, tail_min;
  // Forward 256-row launches: 8 tile-queue counters kTileQueueStride words
  // apart, zero at launch (null: every workgroup takes a fixed share of the tiles).
  int32_t* tileq;
};

constexpr int kMaxSplitParts = 8;  // most K parts of a split tile

// How a launch of ntiles tiles is cut: tiles [0, full) whole (the full rounds of
// split_target workgroups), the rest in sp parts each, part slots in order.
// The GEMM and the reduce kernel derive the same cut from the same plan.
struct SplitCut {
  int64_t full;
  int sp;
};
__device__ __forceinline__ SplitCut split_cut(const GemmArgs& g, int64_t ntiles) {
  if (g.splits <= 1 || ntiles <= 0 || g.split_target <= 0) return {ntiles, 1};
  const int64_t rest = ntiles % g.split_target;
  if (rest == 0) return {ntiles, 1};
  int64_t s = g.split_target / rest;
  if (s > g.splits) s = g.splits;
  if (s * rest > g.partial_cap) s = g.partial_cap / rest;
  if (s < 2 || (ntiles > rest && s < g.tail_min)) return {ntiles, 1};
  return {ntiles - rest, static_cast<int>(s)};
}

// m-block and column block of tile `tile` of a plan-driven launch: tiles run
// group by group (the plan's runs of up to kTileGroup m-blocks of one expert),
// m-block-fastest inside a group; a malformed group entry falls back to a
// group of one.
__device__ __forceinline__ void decode_group_tile(const GemmArgs& g, int64_t tile, int nbc, int nmb, int& mb,
                                                  int& nb) {
  const int row = static_cast<int>(tile / nbc);
  const int info = g.mblocks[row].w;
  int m0 = info >> 4, gs = info & 15;
  if (gs < 1 || gs > kTileGroup || m0 > row || row >= m0 + gs || m0 + gs > nmb) m0 = row, gs = 1;
  const int64_t o = tile - static_cast<int64_t>(m0) * nbc;
  mb = m0 + static_cast<int>(o % gs);
  nb = static_cast<int>(o / gs);
}

// Token of sorted row p (FC1): routed rows through perm, shared rows directly.
__device__ __forceinline__ int64_t row_token(const GemmArgs& g, int64_t p) {
  int64_t tok = p < g.n_routed ? g.perm[p] / g.ktop : (p - g.n_routed) % (g.T > 0 ? g.T : 1);
  return tok < 0 ? 0 : (tok >= g.T ? g.T - 1 : tok);
}

// First weight byte of expert e in a routed tensor B or, for a shared expert, in S.
__device__ __forceinline__ const char* expert_base(const GemmArgs& g, const void* B, const void* S, int e,
                                                   int64_t ebytes) {
  return e < g.E_routed ? static_cast<const char*>(B) + e * ebytes
                        : static_cast<const char*>(S) + static_cast<int64_t>(e - g.E_routed) * ebytes;
}

template <int ACH, int BCH>
__device__ __forceinline__ void gemm_gload(u32x4_t (&ra)[ACH], u32x4_t (&rb)[BCH], const char* const (&aptr)[ACH],
                                           const char* const (&bptr)[BCH], int kt, int rowb) {
  const int64_t koff = static_cast<int64_t>(kt) * rowb;
#pragma unroll
  for (int i = 0; i < ACH; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(aptr[i] + koff);
#pragma unroll
  for (int i = 0; i < BCH; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(bptr[i] + koff);
}

template <int ACH, int BCH, int CPR, int LROW>
__device__ __forceinline__ void gemm_lstore(const u32x4_t (&ra)[ACH], const u32x4_t (&rb)[BCH], char* ldsA, char* ldsB,
                                            const int (&acol)[ACH], const int (&bcol)[BCH], int tid) {
#pragma unroll
  for (int i = 0; i < ACH; ++i)
    *reinterpret_cast<u32x4_t*>(ldsA + ((tid + i * kThreads) / CPR) * LROW + acol[i] * 16) = ra[i];
#pragma unroll
  for (int i = 0; i < BCH; ++i)
    *reinterpret_cast<u32x4_t*>(ldsB + ((tid + i * kThreads) / CPR) * LROW + bcol[i] * 16) = rb[i];
}

template <int kDtype, bool kGated>
__global__ __launch_bounds__(kThreads, kDtype == 1 ? 2 : 1) void grouped_gemm_kernel(GemmArgs g) {
  typedef typename Elt<kDtype>::T T;
  constexpr int EB = Elt<kDtype>::kBytes;
  constexpr int ROWB = kBK * EB;           // bytes per row per K step
  constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  constexpr int LROW = ROWB + 16;          // padded LDS row
  constexpr int ACH = kBM * CPR / kThreads;
  constexpr int BCH = kBNW * CPR / kThreads;
  __shared__ __attribute__((aligned(16))) char lds[(kBM + kBNW) * LROW];
  char* ldsA = lds;
  char* ldsB = lds + kBM * LROW;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t K = g.K, N = g.N;
  const int nmb = g.n_mblocks[0];
  const int nb_count = kGated ? static_cast<int>(N / (kBNW / 2)) : static_cast<int>((N + kBNW - 1) / kBNW);
  const int64_t ntiles = static_cast<int64_t>(nmb) * nb_count;
  const int nk = static_cast<int>(K / kBK);

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int mb = static_cast<int>(tile % nmb);
    const int nb = static_cast<int>(tile / nmb);
    const int4 blk = g.mblocks[mb];
    const int e = blk.x, row0 = blk.y, rows = blk.z;

    // Row pointers of this thread's chunks.
    const char* aptr_[ACH];
    int acol[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / CPR;
      acol[i] = c % CPR;
      const int rr = row0 + (r < rows ? r : 0);
      int64_t arow;
      if constexpr (kGated)
        arow = row_token(g, rr);
      else
        arow = rr;
      aptr_[i] = static_cast<const char*>(g.A) + (arow * K) * EB + acol[i] * 16;
    }
    const char* bptr_[BCH];
    int bcol[BCH];
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / CPR;
      bcol[i] = c % CPR;
      const char* base;
      int64_t n;
      if constexpr (kGated) {
        base = r < kBNW / 2 ? expert_base(g, g.B0, g.S0, e, N * K * EB) : expert_base(g, g.B1, g.S1, e, N * K * EB);
        n = static_cast<int64_t>(nb) * (kBNW / 2) + (r % (kBNW / 2));
      } else {
        base = expert_base(g, g.B0, g.S0, e, N * K * EB);
        n = static_cast<int64_t>(nb) * kBNW + r;
        if (n >= N) n = N - 1;
      }
      bptr_[i] = base + (n * K) * EB + bcol[i] * 16;
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const bool act0 = wm * 64 < rows;
    const bool act1 = wm * 64 + 32 < rows;

    const char* const (&aptr)[ACH] = aptr_;
    const char* const (&bptr)[BCH] = bptr_;
    u32x4_t ra[ACH], rb[BCH];
    gemm_gload<ACH, BCH>(ra, rb, aptr, bptr, 0, ROWB);
    __syncthreads();
    gemm_lstore<ACH, BCH, CPR, LROW>(ra, rb, ldsA, ldsB, acol, bcol, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) gemm_gload<ACH, BCH>(ra, rb, aptr, bptr, kt + 1, ROWB);
      // 4 sub-steps of K = 16; lane half h holds k = 8h .. 8h+7 of each sub-step
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        const int koffb = s * 16 * EB + (lane >> 5) * 8 * EB;
        const int ar0 = wm * 64 + (lane & 31);
        int bro[2];
        if constexpr (kGated) {
          bro[0] = wn * 32 + (lane & 31);
          bro[1] = kBNW / 2 + wn * 32 + (lane & 31);
        } else {
          bro[0] = wn * 64 + (lane & 31);
          bro[1] = wn * 64 + 32 + (lane & 31);
        }
        if constexpr (kDtype == 1) {
          bf16x8_t a[2], b[2];
          a[0] = *reinterpret_cast<const bf16x8_t*>(ldsA + ar0 * LROW + koffb);
          a[1] = *reinterpret_cast<const bf16x8_t*>(ldsA + (ar0 + 32) * LROW + koffb);
          b[0] = *reinterpret_cast<const bf16x8_t*>(ldsB + bro[0] * LROW + koffb);
          b[1] = *reinterpret_cast<const bf16x8_t*>(ldsB + bro[1] * LROW + koffb);
          if (act0) {
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], acc[0][1], 0, 0, 0);
          }
          if (act1) {
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], acc[1][1], 0, 0, 0);
          }
        } else {
          float a[2][8], b[2][8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4* pa0 = reinterpret_cast<const float4*>(ldsA + ar0 * LROW + koffb);
            const float4* pa1 = reinterpret_cast<const float4*>(ldsA + (ar0 + 32) * LROW + koffb);
            const float4* pb = reinterpret_cast<const float4*>(ldsB + bro[h] * LROW + koffb);
            const float4 b0 = pb[0], b1 = pb[1];
            b[h][0] = b0.x; b[h][1] = b0.y; b[h][2] = b0.z; b[h][3] = b0.w;
            b[h][4] = b1.x; b[h][5] = b1.y; b[h][6] = b1.z; b[h][7] = b1.w;
            const float4* pa = h == 0 ? pa0 : pa1;
            const float4 a0 = pa[0], a1 = pa[1];
            a[h][0] = a0.x; a[h][1] = a0.y; a[h][2] = a0.z; a[h][3] = a0.w;
            a[h][4] = a1.x; a[h][5] = a1.y; a[h][6] = a1.z; a[h][7] = a1.w;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (act0) {
              acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0][q], b[0][q], acc[0][0], 0, 0, 0);
              acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0][q], b[1][q], acc[0][1], 0, 0, 0);
            }
            if (act1) {
              acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1][q], b[0][q], acc[1][0], 0, 0, 0);
              acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1][q], b[1][q], acc[1][1], 0, 0, 0);
            }
          }
        }
      }
      __syncthreads();
      if (kt + 1 < nk) {
        gemm_lstore<ACH, BCH, CPR, LROW>(ra, rb, ldsA, ldsB, acol, bcol, tid);
        __syncthreads();
      }
    }

    // Epilogue. Accumulator element v of lane l: row 8*(v/4) + 4*(l/32) + v%4,
    // column l%32 of its 32 x 32 block.
    T* C = static_cast<T*>(g.C);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= rows) continue;
        T* crow = C + static_cast<int64_t>(row0 + r) * N;
        if constexpr (kGated) {
          const int64_t col = static_cast<int64_t>(nb) * (kBNW / 2) + wn * 32 + (lane & 31);
          const float hv = silu_mul(acc[i][0][v], acc[i][1][v]);
          if constexpr (kDtype == 1) crow[col] = static_cast<bf16_t>(f32_to_bf16_bits(hv));
          else crow[col] = hv;
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int64_t col = static_cast<int64_t>(nb) * kBNW + wn * 64 + j * 32 + (lane & 31);
            if (col < N) {
              if constexpr (kDtype == 1) crow[col] = static_cast<bf16_t>(f32_to_bf16_bits(acc[i][j][v]));
              else crow[col] = acc[i][j][v];
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-tile variant for experts with many rows: tile BM x BN, K step 64,
// LDS buffers filled by buffer loads straight into LDS (buffer_load_dwordx4
// ... lds: lane i's 16 bytes land at M0 + 16 * i), 128-byte row segments.
// WM x WN waves, each (BM/WM) x (BN/WN) with 16x16x32 bf16 MFMAs. A has two
// LDS buffers, B three (2 x 32 + 3 x 32 KB: the CU's whole 160 KB). After
// the first of the two 32-wide sub-steps of step kt every wave waits for
// the loads of step kt+1 and meets at the one barrier of the step; step
// kt's buffers are then free, and the loads of A for step kt+2 and of B for
// step kt+3 go out at once (weights, mostly first touches from HBM, get the
// longer lead). The second sub-step's MFMAs hide the LDS reads of step kt+1's
// first sub-step. B fragments alternate between two register sets, one
// sub-step ahead of the MFMAs, and scheduling groups interleave the reads
// and the load issue with the MFMAs.
// On the Mixtral-8x22B prefill FC1 the loop is power-bound: with the loads
// on, the clock settles near 1.6 GHz (2.3 GHz without them), and in cycles
// the kernel runs within about 15 % of the load-free loop.
// LDS rows are BK*2 bytes; the 16-byte chunk c of row r sits in slot
// c ^ f(r), f(r) = (r / R256) mod CPR with R256 = rows per 256 bytes. gfx950's
// LDS has 64 four-byte banks, so a 16-byte-per-lane read is conflict-free when
// every 16 consecutive lanes (16 consecutive rows of a fragment) touch 16
// distinct 16-byte units of a 256-byte line; f spreads them exactly so. The
// swizzle is applied on the load side: the lane filling slot c' of row r
// fetches chunk c' ^ f(r).
// Per-tile buffer descriptors give 32-bit row offsets, keep the K advance in
// the scalar offset, and return zeros outside the tensor (num_records).

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Scheduling pattern for M MFMAs, R LDS reads and V global loads in one basic
// block: max(M, R) groups, MFMAs and reads each spread evenly over them, the
// loads spread over the first VG groups, MFMAs first in every group.
template <int Msk, int Cnt>
__device__ __forceinline__ void sched_group() {
  if constexpr (Cnt > 0) __builtin_amdgcn_sched_group_barrier(Msk, Cnt, 0);
}
template <int M, int R, int V, int VG, int... I>
__device__ __forceinline__ void interleave_mfma_ds_vmem(std::integer_sequence<int, I...>) {
  constexpr int G = sizeof...(I);
  static_assert(G == (M > R ? M : R) && VG >= 1 && VG <= G, "one group per MFMA or LDS read");
  ((sched_group<0x008, ((I + 1) * M) / G - (I * M) / G>(), sched_group<0x100, ((I + 1) * R) / G - (I * R) / G>(),
    sched_group<0x020, (I < VG ? ((I + 1) * V) / VG - (I * V) / VG : 0)>()),
   ...);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Every LDS read of this wave has returned (lgkmcnt 0; vmcnt and expcnt left alone).
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the memory fence __syncthreads() carries: that fence
// makes the compiler wait for every outstanding load, including the LDS stages
// still being prefetched. LDS readiness is handled by explicit vmcnt waits
// before the barrier; the empty asm keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// What a large-tile launch computes. Every form is C = A B^T over 64-wide K
// steps with both operands K-contiguous; they differ in where A rows come
// from, which B rows pair up, and the epilogue.
enum GemmMode : int {
  kModeFc1 = 0,    // h = SiLU(x W1^T) * (x W3^T), A rows gathered by token, bf16 out
  kModeFc2 = 1,    // y = h W2^T, A = the m-block's rows, bf16 out
  kModeFc1GU = 2,  // g | u = x W1^T | x W3^T stored side by side ([rows][2N] bf16), optionally h as well
  kModeBwdQ = 3,   // q = dout W2 (B = W2 as stored, [K][N]), A rows gathered by token, fp32 out
  kModeBwdDx = 4,  // dx rows += dg W1 or du W3 (A = one half of the dg|du rows, B as stored, K = f), fp32 out
  kModeWgrad = 5,  // dW_e = A_e B_e^T, K = expert e's padded rows, fp32 (or bf16) out
};
__host__ __device__ constexpr bool mode_gated(int m) { return m == kModeFc1 || m == kModeFc1GU; }
__host__ __device__ constexpr bool mode_gather(int m) { return m == kModeFc1 || m == kModeFc1GU || m == kModeBwdQ; }
__host__ __device__ constexpr bool mode_f32_out(int m) { return m >= kModeBwdQ; }
// B stored [K][N] (rows N-contiguous): the weights read by the backward's DGrad
__host__ __device__ constexpr bool mode_b_kn(int m) { return m == kModeBwdQ || m == kModeBwdDx; }

// Swizzle of the 16-byte chunks of row k of a [K][256] bf16 LDS stage: chunk c
// of row k sits in slot c ^ f(k). The transposing reads of a B fragment touch
// 16 rows k = 8g + 4h + i (g, i in 0..3) at the same columns; f spreads every
// half-wave over all 64 banks.
__device__ __forceinline__ int kn_swz(int k) { return (k % 4) * 4 + (k / 4) % 4; }

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// One tile of a large-tile GEMM form (the kernel's loop body): tile index ->
// (m-block, n-block), operand descriptors, the pipelined K loop and the
// epilogue. pre(mb) runs once the tile's m-block is known and before any of
// its loads are issued; post(mb) after its results are stored and the tile
// buffer is free again (both no-ops for the standalone kernel).
template <int kMode, int BM, int BN, int WM, int WN, bool kPacked = false>
struct DlGemm {
  static constexpr bool kGated = mode_gated(kMode);
  static constexpr bool kWgrad = kMode == kModeWgrad;
  static constexpr bool kBKN = mode_b_kn(kMode);
  static constexpr int BK = 64;                   // K per step
  static constexpr int RB = BK * 2;               // bytes per LDS row
  static constexpr int CPR = RB / 16;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;            // rows per load instruction
  static constexpr int R256 = 16 / CPR;           // rows per 256 bytes
  static constexpr int NW = WM * WN;              // waves per workgroup
  static constexpr int NT = 64 * NW;              // threads per workgroup
  static constexpr int AI = BM / (NW * RPI);      // A load instructions per wave per stage
  static constexpr int BI = BN / (NW * RPI);      // B load instructions per wave per stage
  static constexpr int LPS = AI + BI;             // loads per thread per stage
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MI = TM / 32;              // 32-row units of the wave's rows (padding granularity)
  static constexpr int MI16 = TM / 16, NJ16 = TN / 16;  // 16 x 16 MFMA blocks of the wave tile
  static constexpr int KS = BK / 32;              // MFMA sub-steps (K = 32) per stage
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(!kGated || (NJ16 % 2 == 0), "gated tiles pair gate and up blocks");
  static_assert(KS == 2, "two 32-wide sub-steps per 64-wide stage");
  static_assert(AI * NW * RPI == BM && BI * NW * RPI == BN, "load tiling");
  static_assert(!kBKN || (BN == 256 && !kGated), "[K][N] weights: 512-byte LDS rows, two per load instruction");
  // LDS: two A buffers, then as many B buffers (up to 8) as fit in the CU's
  // 160 KB, so weight loads run NBB-1 steps ahead
  static constexpr int A_ST = BM * RB, B_ST = BN * RB;
  static constexpr int NBA = 2;
  static constexpr int NBB_FIT = (160 * 1024 - NBA * A_ST) / B_ST;
  static constexpr int NBB = NBB_FIT > 8 ? 8 : NBB_FIT;
  static_assert(NBB >= 2, "two A and two B buffers fit in LDS");
  static constexpr int LDS_BYTES = NBA * A_ST + NBB * B_ST;

  // tiles of one launch: m-blocks (or experts x output-row blocks) x column
  // blocks, times the parts of a split launch
  __device__ static int64_t tiles(const GemmArgs& g) {
    const int64_t N = g.N;
    const int nbc = kGated ? static_cast<int>((N + BN / 2 - 1) / (BN / 2)) : static_cast<int>((N + BN - 1) / BN);
    const int nmb = kWgrad ? g.n_experts * static_cast<int>(g.M / BM) : g.n_mblocks[0];
    const int64_t nt = static_cast<int64_t>(nmb) * nbc;
    if constexpr (kWgrad) return nt;
    const SplitCut c = split_cut(g, nt);
    return c.full + (nt - c.full) * c.sp;
  }

  // Forward tiles of a workgroup can be chained: the last K steps of one tile
  // issue the first loads of the next (into the buffers those steps free), and
  // its epilogue stores straight from registers, so the next tile starts with
  // its first stages already in LDS or in flight. The next tile's load offsets
  // then stay in registers through the whole K loop, which only the 128-row
  // forms have room for (the 256-row ones would spill inside the loop).
  static constexpr bool kChain = (kMode == kModeFc1 || kMode == kModeFc2) && BM == 128;

  // Where a tile's operands come from: its place in the launch, its K steps
  // and the buffer descriptors and per-lane offsets of its A and B loads.
  struct Desc {
    int64_t tile, pslot;
    int sp, part, mb, nb, e, row0, rows, kt0, nk;
    __amdgpu_buffer_rsrc_t ars, brs0, brs1;
    uint32_t aoff[AI], boff[BI];
  };

  template <class Pre, class Post>
  __device__ static __forceinline__ void tile(const GemmArgs& g, char* lds, int64_t vtile, Pre pre, Post post) {
#if defined(__HIP_DEVICE_COMPILE__)
    Desc t;
    describe(g, vtile, t);
    pre(t.mb);  // the tile's operands are ready (fused kernels wait here)
    run_tile(g, lds, t, t, 0, 0, false, post);
#endif
  }

  static constexpr int PH = (RPI / R256) % CPR;  // swizzle phase step per load instruction (0 or 4)
  // Chunk a lane fetches for a load instruction whose first row is R0 (a
  // multiple of RPI): f(R0 + lrow) = (R0 / R256 + lrow / R256) mod CPR, and
  // R0 / R256 mod CPR is 0 for 64-byte rows and 0 or 4 for 128-byte rows
  // (alternating with the instruction index: r0_phase).
  __device__ static __forceinline__ uint32_t chunk_off(int lane, int r0_phase) {
    return static_cast<uint32_t>(((lane % CPR) ^ ((r0_phase + (lane / CPR) / R256) % CPR)) * 16);
  }
  // Forward weights (FC1, FC2; as stored or in stage order): the offset of the
  // 16 bytes load instruction i of wave wv fetches for column block nb.
  // Weights as stored, or (kPacked) in the stage order of pack_weights_kernel:
  // the 64-row group g of an expert's matrix is K / 64 blocks of 8 KiB, block
  // kt holding rows 64g.. x K elements 64kt.. already swizzled as the LDS
  // stage expects, so the lane of stage row r and slot c reads 16 bytes at
  // (g * K/64 + kt) * 8192 + (r % 64) * 128 + c * 16. The stage's column
  // block starts on a multiple of 64 rows, so r % 64 is the row's place in
  // its group and the swizzle matches.
  __device__ static __forceinline__ uint32_t fwd_b_off(const GemmArgs& g, int nb, int i, int wv, int lane) {
    const int64_t K = g.K, N = g.N;
    const int r = (wv * BI + i) * RPI + lane / CPR;
    int64_t n;
    if constexpr (kGated)
      n = static_cast<int64_t>(nb) * (BN / 2) + (r % (BN / 2));
    else
      n = static_cast<int64_t>(nb) * BN + r;
    if constexpr (kPacked) {
      int64_t grp = n / 64;
      if (grp >= N / 64) grp = N / 64 - 1;  // column tail: a valid group, never stored
      return static_cast<uint32_t>(grp * (K / 64) * 8192 + (r % 64) * 128 + (lane % CPR) * 16);
    } else {
      if (n >= N) n = N - 1;  // column tail: computed on a valid row, never stored
      return static_cast<uint32_t>(n * K * 2) + chunk_off(lane, ((wv * BI + i) * PH) % CPR);
    }
  }
  // A rows of a block read in place (FC2 and the other non-gathered forms):
  // row r of `rows` at pitch ap; rows past the end get an offset at the
  // descriptor's size (the load returns zeros and makes no memory request).
  __device__ static __forceinline__ uint32_t plain_a_off(int64_t ap, int rows, int i, int wv, int lane) {
    const uint32_t hb = static_cast<uint32_t>(static_cast<int64_t>(rows) * ap * 2);
    const int r = (wv * AI + i) * RPI + lane / CPR;
    return r < rows ? static_cast<uint32_t>(r * ap * 2) + chunk_off(lane, ((wv * AI + i) * PH) % CPR) : hb;
  }

  __device__ static __forceinline__ void describe(const GemmArgs& g, int64_t vtile, Desc& d) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in a scalar register
    const int64_t K = g.K, N = g.N;
    const int nbc = kGated ? static_cast<int>((N + BN / 2 - 1) / (BN / 2)) : static_cast<int>((N + BN - 1) / BN);
    // weight gradients: every expert has M / BM m-blocks of output rows
    const int mbe = kWgrad ? static_cast<int>(g.M / BM) : 0;
    const int nmb = kWgrad ? g.n_experts * mbe : g.n_mblocks[0];
    int nk = static_cast<int>(K / BK);
    // Virtual tiles: the whole tiles of the full rounds, then the parts of the
    // split tiles, tile-major (part p covers K steps kt0 ..).
    int sp = 1, part = 0;
    int64_t tile = vtile, pslot = 0;
    if constexpr (!kWgrad) {
      const SplitCut c = split_cut(g, static_cast<int64_t>(nmb) * nbc);
      if (vtile >= c.full) {
        sp = c.sp;
        pslot = vtile - c.full;
        tile = c.full + pslot / sp;
        part = static_cast<int>(pslot % sp);
      }
    }
    int kt0 = 0;
    const int lrow = lane / CPR;                                          // row within a load instruction
    auto chunk_off = [&](int r0_phase) -> uint32_t { return DlGemm::chunk_off(lane, r0_phase); };
    // x spans T*K*2 bytes (< 2^32, checked on the host)
    const uint32_t a_bytes = mode_gather(kMode) ? static_cast<uint32_t>(g.T * K * 2) : 0u;

    int mb, nb, e, row0, rows;
    __amdgpu_buffer_rsrc_t ars;
    uint32_t aoff[AI];
    if constexpr (kWgrad) {
      // expert-major, m-block fastest: neighbouring tiles share a B panel
      const int64_t per_e = static_cast<int64_t>(mbe) * nbc;
      e = static_cast<int>(tile / per_e);
      const int r = static_cast<int>(tile % per_e);
      mb = r % mbe;
      nb = r / mbe;
      const int k0 = g.kofs[e], k1 = g.kofs[e + 1];
      nk = (k1 - k0) / BK;
      row0 = mb * BM;
      rows = BM;
      // A_e: rows row0.. of the transposed operand, K window from column k0
      const uint32_t bytes = static_cast<uint32_t>((g.M * g.pitch - k0) * 2);
      ars = make_rsrc(static_cast<const char*>(g.A) + static_cast<int64_t>(k0) * 2, bytes);
#pragma unroll
      for (int i = 0; i < AI; ++i) {
        const int r2 = (wv * AI + i) * RPI + lrow;
        aoff[i] = static_cast<uint32_t>((row0 + r2) * g.pitch * 2) + chunk_off(((wv * AI + i) * PH) % CPR);
      }
    } else {
      decode_group_tile(g, tile, nbc, nmb, mb, nb);
      if (sp > 1) {
        kt0 = static_cast<int>(static_cast<int64_t>(part) * nk / sp);
        nk = static_cast<int>(static_cast<int64_t>(part + 1) * nk / sp) - kt0;
      }
      const int4 blk = g.mblocks[mb];
      e = __builtin_amdgcn_readfirstlane(blk.x);
      row0 = __builtin_amdgcn_readfirstlane(blk.y);
      rows = __builtin_amdgcn_readfirstlane(blk.z);

      // A: FC1 gathers token rows of x; FC2 reads rows row0.. of h. Rows past the
      // block's end get an offset at the descriptor's size: the load returns zeros
      // and makes no memory request.
      if constexpr (mode_gather(kMode)) {
        ars = make_rsrc(g.A, a_bytes);
#pragma unroll
        for (int i = 0; i < AI; ++i) {
          const int r = (wv * AI + i) * RPI + lrow;
          if (r < rows) {
            const int64_t tok = row_token(g, row0 + r);
            aoff[i] = static_cast<uint32_t>(tok * K * 2) + chunk_off(((wv * AI + i) * PH) % CPR);
          } else {
            aoff[i] = a_bytes;
          }
        }
      } else {
        const int64_t ap = g.a_pitch > 0 ? g.a_pitch : K;  // row pitch of A (elements)
        const uint32_t hb = static_cast<uint32_t>(static_cast<int64_t>(rows) * ap * 2);
        ars = make_rsrc(static_cast<const char*>(g.A) + (static_cast<int64_t>(row0) * ap + g.a_col0) * 2, hb);
#pragma unroll
        for (int i = 0; i < AI; ++i) aoff[i] = plain_a_off(ap, rows, i, wv, lane);
      }
    }

    // B: weight rows of expert e (gated: first half W1, second half W3, same
    // columns); weight gradients: rows of the transposed operand, K window of expert e.
    __amdgpu_buffer_rsrc_t brs0, brs1;
    uint32_t boff[BI];
    if constexpr (kBKN) {
      // [K][N] weights (DGrad reads them as stored): a stage is BK rows of BN
      // columns, 512 bytes per row, two rows per load instruction; the lane that
      // fills slot c' of row r fetches chunk c' ^ f(r).
      const int64_t ebytes = K * N * 2;
      brs0 = make_rsrc(expert_base(g, g.B0, g.S0, e, ebytes), static_cast<uint32_t>(ebytes));
      brs1 = brs0;
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int r = 2 * (wv * BI + i) + lane / 32;  // stage row of this lane's 16 bytes
        boff[i] = static_cast<uint32_t>(static_cast<int64_t>(r) * N * 2 + static_cast<int64_t>(nb) * BN * 2 +
                                        ((lane % 32) ^ kn_swz(r)) * 16);
      }
    } else if constexpr (kWgrad) {
      const int k0 = g.kofs[e];
      brs0 = make_rsrc(static_cast<const char*>(g.B0) + static_cast<int64_t>(k0) * 2,
                       static_cast<uint32_t>((N * g.pitch - k0) * 2));
      brs1 = brs0;
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int r = (wv * BI + i) * RPI + lrow;
        boff[i] = static_cast<uint32_t>((static_cast<int64_t>(nb) * BN + r) * g.pitch * 2) +
                  chunk_off(((wv * BI + i) * PH) % CPR);
      }
    } else {
      // forward weights (fwd_b_off)
      const int64_t ebytes = N * K * 2;
      brs0 = make_rsrc(expert_base(g, g.B0, g.S0, e, ebytes), static_cast<uint32_t>(ebytes));
      brs1 = kGated ? make_rsrc(expert_base(g, g.B1, g.S1, e, ebytes), static_cast<uint32_t>(ebytes)) : brs0;
#pragma unroll
      for (int i = 0; i < BI; ++i) boff[i] = fwd_b_off(g, nb, i, wv, lane);
    }

    d.tile = tile;
    d.pslot = pslot;
    d.sp = sp;
    d.part = part;
    d.mb = mb;
    d.nb = nb;
    d.e = e;
    d.row0 = row0;
    d.rows = rows;
    d.kt0 = kt0;
    d.nk = nk;
    d.ars = ars;
    d.brs0 = brs0;
    d.brs1 = brs1;
#pragma unroll
    for (int i = 0; i < AI; ++i) d.aoff[i] = aoff[i];
#pragma unroll
    for (int i = 0; i < BI; ++i) d.boff[i] = boff[i];
#endif
  }

  // The K loop and epilogue of tile t. s0: index of the tile's first K step in
  // the workgroup's sequence of steps (step s uses A buffer s % 2 and B buffer
  // s % NBB). warm: the previous tile's last steps already issued t's first
  // loads. nx: the next tile, whose first nx_nk steps' loads this tile's last
  // steps issue (nx_nk = 0: none; those steps then load nothing).
  template <class Post>
  __device__ static __forceinline__ void run_tile(const GemmArgs& g, char* lds, const Desc& t, const Desc& nx,
                                                  int nx_nk, int s0, bool warm, Post post) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in a scalar register
    const int wm = wv / WN, wn = wv % WN;
    const int64_t N = g.N;
    const int fsw = ((lane & 15) / R256) % CPR;  // read-side swizzle of row (lane & 15)
    const int64_t pslot = t.pslot;
    const int sp = t.sp, mb = t.mb, nb = t.nb, e = t.e, row0 = t.row0, rows = t.rows, kt0 = t.kt0, nk = t.nk;
    const bool chained = kChain && nx_nk > 0;
    const __amdgpu_buffer_rsrc_t ars = t.ars, brs0 = t.brs0, brs1 = t.brs1;
    const uint32_t(&aoff)[AI] = t.aoff;
    const uint32_t(&boff)[BI] = t.boff;

    f32x4_t acc[MI16][NJ16];
#pragma unroll
    for (int i = 0; i < MI16; ++i)
#pragma unroll
      for (int j = 0; j < NJ16; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

    // Loads of K step kt into LDS slot `stage`. Steps past the end load from an
    // empty descriptor (zeros, no memory access) into a slot nobody reads
    // again, so every step issues the same number of loads and the issue can
    // sit in the same basic block as the MFMAs.
    const __amdgpu_buffer_rsrc_t nul = make_rsrc(g.B0, 0u);
    constexpr uint32_t kstride = kPacked ? 8192u : static_cast<uint32_t>(RB);  // B bytes per K step
    auto issue_a = [&](int slot, int kt) {
      const bool real = kt < nk;
      char* sa = lds + slot * A_ST;
      if constexpr (kChain) {
        // past the tile's end: step kt - nk of the next tile, if any
        const int kn = kt - nk;
        const bool ahead = !real && chained && kn < nx_nk;
        const __amdgpu_buffer_rsrc_t rs = real ? ars : (ahead ? nx.ars : nul);
        const uint32_t koff = static_cast<uint32_t>(real ? kt0 + kt : (ahead ? nx.kt0 + kn : 0)) * RB;
#pragma unroll
        for (int i = 0; i < AI; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(sa + (wv * AI + i) * 1024),
                                                   16, real ? aoff[i] : nx.aoff[i], koff, 0, 0);
        return;
      }
      const uint32_t koff = real ? static_cast<uint32_t>(kt0 + kt) * RB : 0u;
#pragma unroll
      for (int i = 0; i < AI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            real ? ars : nul, (__attribute__((address_space(3))) void*)(sa + (wv * AI + i) * 1024), 16, aoff[i],
            koff, 0, 0);
    };
    // aux_c: cache policy of the weight loads (0, or 2 = non-temporal)
    auto issue_b = [&](int slot, int kt, auto aux_c) {
      constexpr int AUX = decltype(aux_c)::value;
      const bool real = kt < nk;
      char* sb = lds + NBA * A_ST + slot * B_ST;
      if constexpr (kBKN) {
        // step kt is weight rows kt*BK..
        const uint32_t koff = real ? static_cast<uint32_t>(kt0 + kt) * static_cast<uint32_t>(BK * N * 2) : 0u;
#pragma unroll
        for (int i = 0; i < BI; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(real ? brs0 : nul,
                                                   (__attribute__((address_space(3))) void*)(sb + (wv * BI + i) * 1024),
                                                   16, boff[i], koff, 0, AUX);
        return;
      }
      if constexpr (kChain) {
        const int kn = kt - nk;
        const bool ahead = !real && chained && kn < nx_nk;
        const __amdgpu_buffer_rsrc_t r0 = real ? brs0 : (ahead ? nx.brs0 : nul);
        const __amdgpu_buffer_rsrc_t r1 = real ? brs1 : (ahead ? nx.brs1 : nul);
        const uint32_t koff = static_cast<uint32_t>(real ? kt0 + kt : (ahead ? nx.kt0 + kn : 0)) * kstride;
#pragma unroll
        for (int i = 0; i < BI; ++i) {
          const bool second = kGated && ((wv * BI + i) * RPI >= BN / 2);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? r1 : r0,
                                                   (__attribute__((address_space(3))) void*)(sb + (wv * BI + i) * 1024),
                                                   16, real ? boff[i] : nx.boff[i], koff, 0, AUX);
        }
        return;
      }
      // (steps past the end read through the empty descriptor: the offset is moot)
      const uint32_t koff = static_cast<uint32_t>(kt0 + kt) * kstride;
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const bool second = kGated && ((wv * BI + i) * RPI >= BN / 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            real ? (second ? brs1 : brs0) : nul, (__attribute__((address_space(3))) void*)(sb + (wv * BI + i) * 1024),
            16, boff[i], koff, 0, AUX);
      }
    };
    // bf16 MFMA 16x16x32 (under a sustained power limit it keeps a higher
    // rate than 32x32x16: half the accumulator traffic per FLOP). Lane l holds
    // row l % 16 and K elements 8 * (l / 16) .. +7 of an A or B fragment, and
    // rows 4 * (l / 16) .. +3 of column l % 16 of the 16 x 16 result.
    // Only the wave's first MA 32-row units hold rows of the m-block; the
    // others are padding, so their fragments are neither read nor multiplied
    // (their accumulators stay zero and are never stored).
    // Fragments: fb[set] double-buffered per 32-wide sub-step; fa[i] refilled
    // with the next sub-step's row block i as soon as block i's MFMAs are issued.
    bf16x8_t fa[MI16], fb[2][NJ16];
    auto ck_of = [&](int s) { return (((4 * s + (lane >> 4)) ^ fsw) % CPR) * 16; };
    auto read_a = [&](int i, int s, int a_slot) {
      const char* sa = lds + a_slot * A_ST;
      fa[i] = *reinterpret_cast<const bf16x8_t*>(sa + (wm * TM + 16 * i + (lane & 15)) * RB + ck_of(s));
    };
    auto read_b = [&](int set, int s, int b_slot) {
      const char* sb = lds + NBA * A_ST + b_slot * B_ST;
      if constexpr (kBKN) {
        // Transposing reads (ds_read_b64_tr_b16): in each group of 16 lanes,
        // lane 16g + 4i + q reads 4 columns 4q.. of row k = 8g + 4h + i, and the
        // instruction hands lane l the column l % 16 of rows 8(l / 16) + 4h + 0..3:
        // two reads (h = 0, 1) give the fragment's 8 K values of one column.
        // Per lane: row k0 = 8g + 4h + i of the 32-row sub-step, the byte within
        // the 16-byte chunk, and the row's swizzle (f(32s + k0) = f(k0)).
#pragma unroll
        for (int j = 0; j < NJ16; ++j) {
          const int c = (wn * TN + 16 * j) / 8 + (lane % 4) / 2;  // 16-byte chunk of the lane's 4 columns
          i16x4_t half[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int k0 = 8 * (lane / 16) + 4 * h + (lane % 16) / 4;
            const char* p = sb + s * (32 * 512) + k0 * 512 + (lane % 2) * 8 + ((c ^ kn_swz(k0)) & 31) * 16;
            half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
          }
          fb[set][j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
        return;
      }
#pragma unroll
      for (int j = 0; j < NJ16; ++j) {
        int brow;
        if constexpr (kGated)
          brow = (j < NJ16 / 2 ? 0 : BN / 2) + wn * (TN / 2) + 16 * (j % (NJ16 / 2)) + (lane & 15);
        else
          brow = wn * TN + 16 * j + (lane & 15);
        fb[set][j] = *reinterpret_cast<const bf16x8_t*>(sb + brow * RB + ck_of(s));
      }
    };
    // MFMAs of sub-step `set` over the first MA16 row blocks, each block's A
    // fragment then refilled with sub-step ns of A buffer a_slot
    auto mfma_refill = [&](auto ma_c, int set, int ns, int a_slot) {
      constexpr int MA16 = 2 * decltype(ma_c)::value < MI16 ? 2 * decltype(ma_c)::value : MI16;
#pragma unroll
      for (int i = 0; i < MA16; ++i) {
#pragma unroll
        for (int j = 0; j < NJ16; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[set][j], acc[i][j], 0, 0, 0);
        read_a(i, ns, a_slot);
      }
    };

    auto kloop = [&](auto ma_c, auto aux_c) {
      constexpr int MA16 = 2 * decltype(ma_c)::value < MI16 ? 2 * decltype(ma_c)::value : MI16;
      // Step j uses A buffer j & 1 and B buffer j % NBB; both are free once
      // every wave passed step j's barrier (its reads are done by then), so
      // the loads of A for step j+2 and of B for step j+NBB are issued right
      // there, in that order. vmcnt counts in issue order, so the prologue
      // issues as the steps before step 0 would have: B0 .. B(NBB-3), A0,
      // B(NBB-2), A1, B(NBB-1) (two buffers: B0 A0 A1 B1). At step kt's
      // barrier only the newest B batch, B(kt+NBB-1), may then be in flight.
      // Buffers of the tile's step 0 (step j uses A buffer (a0 + j) % 2 and B
      // buffer (b0 + j) % NBB). A warm tile's loads of steps 0 .. NBB-1 (A:
      // 0, 1) went out in that order during the previous tile's last steps;
      // only the epilogue's stores can be newer, and they only make the wait
      // below longer.
      const int a0 = s0 & 1, b0 = s0 % NBB;
      auto bslot = [&](int j) { return b0 + j < NBB ? b0 + j : b0 + j - NBB; };
      if (!warm) {
        if constexpr (NBB == 2) {
          issue_b(bslot(0), 0, aux_c);
          issue_a(a0, 0);
          issue_a(a0 ^ 1, 1);
          issue_b(bslot(1), 1, aux_c);
        } else {
          issue_b(bslot(0), 0, aux_c);
#pragma unroll
          for (int j = 1; j <= NBB - 3; ++j) issue_b(bslot(j), j, aux_c);
          issue_a(a0, 0);
          issue_b(bslot(NBB - 2), NBB - 2, aux_c);
          issue_a(a0 ^ 1, 1);
          issue_b(bslot(NBB - 1), NBB - 1, aux_c);
        }
      }
      wait_vmcnt<(NBB == 2 ? AI + BI : AI + 2 * BI)>();  // A0 and B0 landed
      lds_barrier();
      if constexpr (MA16 > 0) {
        read_b(0, 0, b0);
#pragma unroll
        for (int i = 0; i < MA16; ++i) read_a(i, 0, a0);
      }
      int bsl = b0;  // B buffer of step kt
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = (a0 + kt) & 1;
        const int bnx = bsl + 1 == NBB ? 0 : bsl + 1;
        constexpr int M = MA16 * NJ16, R = MA16 + NJ16, G = M > R ? M : R;
        if constexpr (MA16 > 0) {
          // sub-step 0: its MFMAs with the reads of sub-step 1 (same buffers)
          read_b(1, 1, bsl);
          mfma_refill(ma_c, 0, 1, cur);
          interleave_mfma_ds_vmem<M, R, 0, 1>(std::make_integer_sequence<int, G>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmcnt<(NBB == 2 ? 0 : BI)>();  // this thread's loads of step kt+1 landed
        wait_lds_reads();  // and its reads of step kt's buffers are done: they may be refilled after the barrier
        lds_barrier();
        issue_a(cur, kt + 2);
        issue_b(bsl, kt + NBB, aux_c);
        if constexpr (MA16 > 0) {
          // sub-step 1: its MFMAs with the reads of step kt+1's sub-step 0
          // (on the last step: zeros, unused)
          read_b(0, 0, bnx);
          mfma_refill(ma_c, 1, 0, cur ^ 1);
          interleave_mfma_ds_vmem<M, R, LPS, G>(std::make_integer_sequence<int, G>{});
        }
        __builtin_amdgcn_sched_barrier(0);
        bsl = bnx;
      }
      // the loads of the last steps (the next tile's, or empty ones) still write
      // LDS: an epilogue through LDS waits for them, one from registers does not
      if (!(kChain && sp == 1)) wait_vmcnt<0>();
    };

    const int ma = __builtin_amdgcn_readfirstlane(min(MI, max(0, (rows - wm * TM + 31) / 32)));
    auto run = [&](auto aux_c) {
      if (ma >= MI) {
        kloop(std::integral_constant<int, MI>{}, aux_c);
      } else {
        static_assert(MI <= 4, "active-block dispatch covers up to four 32-row blocks per wave");
        switch (ma) {
          case 0: kloop(std::integral_constant<int, 0>{}, aux_c); break;
          case 1: kloop(std::integral_constant<int, (MI > 1 ? 1 : MI)>{}, aux_c); break;
          case 2: kloop(std::integral_constant<int, (MI > 2 ? 2 : MI)>{}, aux_c); break;
          default: kloop(std::integral_constant<int, (MI > 3 ? 3 : MI)>{}, aux_c); break;
        }
      }
    };
    // Forward weight tiles of an m-block that is alone in its plan group (an
    // expert with at most one block of rows, as in decode batches) are read by
    // this tile only: they are streamed with the non-temporal cache policy,
    // which sustains a higher HBM read rate. Weights that the neighbouring
    // m-blocks of a group read again keep the default policy, under which the
    // other reads hit in L2.
    if constexpr (kMode == kModeFc1 || kMode == kModeFc2) {
      if ((g.mblocks[mb].w & 15) == 1)
        run(std::integral_constant<int, 2>{});
      else
        run(std::integral_constant<int, 0>{});
    } else {
      run(std::integral_constant<int, 0>{});
    }

    if (mode_f32_out(kMode) || sp > 1) {
      // fp32 epilogue through LDS, IG 16-row blocks i of every wave's rows at a
      // time (so the accumulators of those blocks die as they are stored): the
      // waves write acc[i] into [IG][WM * 16][BN + 4] tiles (the 4-float pad
      // spreads a fragment's 4-row steps over distinct banks), then all threads
      // store 16-byte row chunks.
      constexpr int CP = BN + 4;
      constexpr int SR = WM * 16;  // rows per slice
      static_assert(SR * CP * 4 <= LDS_BYTES, "slice fits in the stage buffers");
      float* ct = reinterpret_cast<float*>(lds);
      // destination: rows of pitch cp from column col0, ncols columns in all
      float* cbase;
      bf16_t* hbase = nullptr;  // weight gradients stored as bf16
      int64_t cp = N, col0 = static_cast<int64_t>(nb) * BN, ncols = N;
      if (sp > 1) {
        // one part of a split tile: the raw accumulators, [BM][BN]
        cbase = g.partial + pslot * (BM * BN);
        cp = BN, col0 = 0, ncols = BN;
      } else if constexpr (kWgrad) {
        const int64_t m0 = static_cast<int64_t>(row0);
        const bool second = m0 >= g.split;
        const int64_t off = static_cast<int64_t>(e) * g.split * N + (second ? m0 - g.split : m0) * N;
        cbase = static_cast<float*>(second ? g.C2 : g.C) + off;
        if (g.out_bf16) hbase = static_cast<bf16_t*>(second ? g.C2 : g.C) + off;
      } else {
        cbase = static_cast<float*>(g.C) + static_cast<int64_t>(row0) * N;
      }
      constexpr int VPR = BN / 4;  // 16-byte vectors per tile row
      if (kWgrad && hbase != nullptr) {
        // bf16 weight gradients: the whole tile at once, rounded into a
        // [BM][BN + 8] bf16 tile (the pad spreads a fragment's 4-row steps
        // over distinct banks), then 8 columns per 16-byte store
        constexpr int HP = BN + 8, VPR8 = BN / 8;
        static_assert(BM * HP * 2 <= LDS_BYTES, "bf16 tile fits in the stage buffers");
        bf16_t* ht = reinterpret_cast<bf16_t*>(lds);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < MI16; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int j = 0; j < NJ16; ++j)
              ht[(wm * TM + 16 * i + 4 * (lane >> 4) + v) * HP + wn * TN + 16 * j + (lane & 15)] =
                  static_cast<bf16_t>(f32_to_bf16_bits(acc[i][j][v]));
        __syncthreads();
        for (int q = tid; q < rows * VPR8; q += NT) {
          const int r = q / VPR8, c8 = (q % VPR8) * 8;
          if (col0 + c8 < ncols)
            *reinterpret_cast<u32x4_t*>(hbase + static_cast<int64_t>(r) * cp + col0 + c8) =
                *reinterpret_cast<const u32x4_t*>(ht + r * HP + c8);
        }
      } else {
        // IG blocks i per pass: as many as fit in the stage buffers for the
        // backward's fp32 forms (fewer barriers), one for the forward's split parts
        constexpr int IG = (mode_f32_out(kMode) && MI16 % 4 == 0 && 4 * SR * CP * 4 <= LDS_BYTES) ? 4 : 1;
#pragma unroll
        for (int i0 = 0; i0 < MI16; i0 += IG) {
          lds_barrier();
#pragma unroll
          for (int ii = 0; ii < IG; ++ii)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
              for (int j = 0; j < NJ16; ++j)
                ct[(ii * SR + wm * 16 + 4 * (lane >> 4) + v) * CP + wn * TN + 16 * j + (lane & 15)] =
                    acc[i0 + ii][j][v];
          __syncthreads();
          for (int q = tid; q < IG * SR * VPR; q += NT) {
            const int rl = q / VPR, c4 = (q % VPR) * 4;
            const int rs = rl % SR;
            const int r = (rs / 16) * TM + 16 * (i0 + rl / SR) + rs % 16;  // row of the tile
            if (r < rows && col0 + c4 < ncols) {
              f32x4_t* dst = reinterpret_cast<f32x4_t*>(cbase + static_cast<int64_t>(r) * cp + col0 + c4);
              const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ct + rl * CP + c4);
              *dst = (g.accumulate && sp == 1) ? *dst + v : v;
            }
          }
        }
      }
    } else if constexpr (kChain) {
      // FC1 / FC2 outputs straight from the accumulators (the stage buffers may
      // already hold the next tile's first steps): lane l holds rows
      // 4 (l / 16) .. +3 of column l % 16 of each 16 x 16 block; FC1 stores
      // SiLU(g) * u of its gate and up blocks.
      bf16_t* C = static_cast<bf16_t*>(g.C);
      constexpr int CJ = kGated ? NJ16 / 2 : NJ16;  // output column blocks of the wave
      const int64_t col0 = static_cast<int64_t>(nb) * (kGated ? BN / 2 : BN) + wn * (kGated ? TN / 2 : TN) + (lane & 15);
#pragma unroll
      for (int i = 0; i < MI16; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = wm * TM + 16 * i + 4 * (lane >> 4) + v;
          if (r < rows) {
            bf16_t* crow = C + static_cast<int64_t>(row0 + r) * N;
#pragma unroll
            for (int j = 0; j < CJ; ++j) {
              const int64_t col = col0 + 16 * j;
              const float val = kGated ? silu_mul(acc[i][j][v], acc[i][j + NJ16 / 2][v]) : acc[i][j][v];
              if (col < N) crow[col] = static_cast<bf16_t>(f32_to_bf16_bits(val));
            }
          }
        }
      }
    } else {
      // Epilogue through LDS: every wave writes its fragment values (bf16) into a
      // row-major [BM][CW] tile, then all threads store whole 16-byte row chunks.
      // The recompute form keeps g and u apart: columns 0..BN/2-1 of the tile
      // are g, the rest u, stored to the two halves of a [rows][2N] row.
      constexpr int CW = (kGated && kMode != kModeFc1GU) ? BN / 2 : BN;  // output columns of the tile
      static_assert(BM * CW * 2 <= LDS_BYTES, "epilogue tile fits in the stage buffers");
      lds_barrier();
      bf16_t* ct = reinterpret_cast<bf16_t*>(lds);
      if constexpr (kMode == kModeFc1GU) {
        if (g.C2 != nullptr) {
          // h = SiLU(g) u from the fp32 accumulators, as the plain FC1 forms
          // it, in a pass of its own ([BM][BN/2] through the same buffer)
          constexpr int HW = BN / 2, HPR = HW / 8;
#pragma unroll
          for (int i = 0; i < MI16; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int r = wm * TM + 16 * i + 4 * (lane >> 4) + v;
#pragma unroll
              for (int j = 0; j < NJ16 / 2; ++j) {
                const int c = wn * (TN / 2) + 16 * j + (lane & 15);
                ct[r * HW + c] = static_cast<bf16_t>(f32_to_bf16_bits(silu_mul(acc[i][j][v], acc[i][j + NJ16 / 2][v])));
              }
            }
          }
          __syncthreads();
          bf16_t* H = static_cast<bf16_t*>(g.C2);
          const int64_t col0 = static_cast<int64_t>(nb) * HW;
          for (int q = tid; q < rows * HPR; q += NT) {
            const int r = q / HPR, c8 = (q % HPR) * 8;
            if (col0 + c8 < N)
              *reinterpret_cast<u32x4_t*>(H + static_cast<int64_t>(row0 + r) * N + col0 + c8) =
                  *reinterpret_cast<const u32x4_t*>(ct + r * HW + c8);
          }
          __syncthreads();  // h is read out before g | u refill the buffer
        }
      }
#pragma unroll
      for (int i = 0; i < MI16; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = wm * TM + 16 * i + 4 * (lane >> 4) + v;
          if constexpr (kMode == kModeFc1GU) {
#pragma unroll
            for (int j = 0; j < NJ16 / 2; ++j) {
              const int c = wn * (TN / 2) + 16 * j + (lane & 15);
              ct[r * CW + c] = static_cast<bf16_t>(f32_to_bf16_bits(acc[i][j][v]));
              ct[r * CW + BN / 2 + c] = static_cast<bf16_t>(f32_to_bf16_bits(acc[i][j + NJ16 / 2][v]));
            }
          } else if constexpr (kGated) {
#pragma unroll
            for (int j = 0; j < NJ16 / 2; ++j) {
              const int c = wn * (TN / 2) + 16 * j + (lane & 15);
              ct[r * CW + c] = static_cast<bf16_t>(f32_to_bf16_bits(silu_mul(acc[i][j][v], acc[i][j + NJ16 / 2][v])));
            }
          } else {
#pragma unroll
            for (int j = 0; j < NJ16; ++j) {
              const int c = wn * TN + 16 * j + (lane & 15);
              ct[r * CW + c] = static_cast<bf16_t>(f32_to_bf16_bits(acc[i][j][v]));
            }
          }
        }
      }
      __syncthreads();
      {
        bf16_t* C = static_cast<bf16_t*>(g.C);
        constexpr int VPR = CW / 8;  // 16-byte vectors per tile row
        if constexpr (kMode == kModeFc1GU) {
          const int64_t col0 = static_cast<int64_t>(nb) * (BN / 2);
          for (int q = tid; q < rows * VPR; q += NT) {
            const int r = q / VPR, c8 = (q % VPR) * 8;
            const int cc = c8 % (BN / 2);
            if (col0 + cc < N)
              *reinterpret_cast<u32x4_t*>(C + static_cast<int64_t>(row0 + r) * 2 * N + (c8 >= BN / 2 ? N : 0) + col0 + cc) =
                  *reinterpret_cast<const u32x4_t*>(ct + r * CW + c8);
          }
        } else {
          const int64_t col0 = static_cast<int64_t>(nb) * CW;
          for (int q = tid; q < rows * VPR; q += NT) {
            const int r = q / VPR, c8 = (q % VPR) * 8;
            if (col0 + c8 < N)
              *reinterpret_cast<u32x4_t*>(C + static_cast<int64_t>(row0 + r) * N + col0 + c8) =
                  *reinterpret_cast<const u32x4_t*>(ct + r * CW + c8);
          }
        }
      }
    }
    __syncthreads();  // the tile buffer is read out before the next tile's loads refill the stages
    post(mb);
#endif
  }
};

// A value every lane holds the same, moved to scalar registers (the compiler
// cannot tell that a word read from LDS is uniform).
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int kMode, int BM, int BN, int WM, int WN, bool kPacked = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_dl_kernel(GemmArgs g) {
  // device-only body: the buffer-resource builtins have no host form, and the
  // host pass only needs the kernel's launch stub
#if defined(__HIP_DEVICE_COMPILE__)
  using D = DlGemm<kMode, BM, BN, WM, WN, kPacked>;
  __shared__ __attribute__((aligned(1024))) char lds[D::LDS_BYTES];
  const int64_t ntiles = D::tiles(g);
  // Workgroups are dealt round-robin to the 8 XCDs (workgroup b runs on XCD
  // b % 8). Renumber so that the gridDim/8 workgroups of one XCD take
  // consecutive tiles of each round, which share A and B blocks in that XCD's L2.
  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  if constexpr (D::kChain) {
    // whole tiles chained: each one's last steps issue the next one's first loads
    typename D::Desc cur, nxt;
    int s0 = 0;
    bool warm = false;
    if (slot < ntiles) D::describe(g, slot, cur);
    for (int64_t tile = slot; tile < ntiles; tile += G) {
      const bool more = tile + G < ntiles;
      if (more) D::describe(g, tile + G, nxt);
      // a tile's last steps issue loads up to NBB steps ahead: all of them must
      // fall in the next tile (so it needs at least NBB steps)
      const bool chain = more && cur.sp == 1 && nxt.sp == 1 && nxt.nk >= D::NBB;
      D::run_tile(g, lds, cur, nxt, chain ? nxt.nk : 0, s0, warm, [](int) {});
      s0 = chain ? s0 + cur.nk : 0;
      warm = chain;
      cur = nxt;
    }
  } else if (g.tileq != nullptr && G % 8 == 0 && g.n_mblocks[kPlanMulti] != 0) {
    // Tile queues, where some expert's rows span several m-blocks (else the
    // tiles are of one length, the weights streamed once, and the fixed
    // shares below measured faster). Tiles of unequal length (partial
    // m-blocks, the K parts of a last round) leave CUs and whole XCDs idle at
    // the end of a launch whose workgroups each take a fixed share. Queue q
    // lists, round by round, the tiles the fixed order gives XCD q (G/8
    // consecutive ones, which share operand panels in that L2); a workgroup
    // takes the next tile of its own XCD's queue and, once that is drained,
    // of the other queues. A queue's tile index grows with its counter, so a
    // queue seen drained stays drained, and every tile is taken once.
    const int per = G / 8;
    int q = blockIdx.x % 8, left = 8;  // used by thread 0 only
    int64_t* bcast = reinterpret_cast<int64_t*>(lds);  // free between tiles
    for (;;) {
      if (threadIdx.x == 0) {
        int64_t t = -1;
        while (left > 0) {
          const int i = atomicAdd(g.tileq + q * kTileQueueStride, 1);
          const int64_t cand = static_cast<int64_t>(i / per) * G + q * per + i % per;
          if (i >= 0 && cand < ntiles) {  // (a counter that is not a claim count reads as drained)
            t = cand;
            break;
          }
          q = (q + 1) % 8;
          --left;
        }
        *bcast = t;
      }
      __syncthreads();
      // the same in every lane: held in scalar registers, as the fixed order's
      // index is (buffer descriptors derived from it must be scalar)
      const int64_t tile = uniform(*reinterpret_cast<volatile int64_t*>(bcast));
      __syncthreads();  // read by every thread before the tile's loads refill the buffer
      if (tile < 0) break;
      D::tile(g, lds, tile, [](int) {}, [](int) {});
    }
  } else {
    for (int64_t tile = slot; tile < ntiles; tile += G) D::tile(g, lds, tile, [](int) {}, [](int) {});
  }
#endif
}

// Second half of a split launch for split tile t (t >= cut.full): per output
// element, the sum of its parts in part order, then what the GEMM's bf16
// epilogue applies: SiLU(g) * u for FC1 (a wave's TN accumulator columns hold
// TN/2 gate columns then the TN/2 up columns of the same outputs), bf16
// rounding. Threads tid, tid + nthr, ... of the caller share the tile, four
// output columns each step (16-byte loads of every part, all issued before
// the sums; N is a multiple of 64, so a group of four is wholly inside or
// outside the matrix).
template <bool kGated, int BM, int BN, int WN>
__device__ __forceinline__ void reduce_split_tile(const GemmArgs& g, int64_t t, SplitCut cut, int nbc, int nmb,
                                                  int tid, int nthr) {
  constexpr int OC = kGated ? BN / 2 : BN;  // output columns of a tile
  constexpr int TN = BN / WN;
  constexpr int OV = OC / 4;                // groups of four output columns
  static_assert(OC % 4 == 0 && (TN / 2) % 4 == 0, "four columns never straddle a gate/up boundary");
  const int64_t N = g.N;
  const int sp = cut.sp;  // at most kMaxSplitParts
  bf16_t* C = static_cast<bf16_t*>(g.C);
  int mb, nb;
  decode_group_tile(g, t, nbc, nmb, mb, nb);
  const int4 blk = g.mblocks[mb];
  const int row0 = blk.y, rows = blk.z;
  const float* part = g.partial + (t - cut.full) * sp * (BM * BN);
  // (an opaque copy of the thread index keeps the compiler from hoisting this
  // loop's index arithmetic out of a caller's tile loop, where it would hold
  // registers through the GEMM)
  asm volatile("" : "+v"(tid));
  for (int q = tid; q < rows * OV; q += nthr) {
    const int r = q / OV, oc = (q % OV) * 4;
    const int64_t col = static_cast<int64_t>(nb) * OC + oc;
    if (col >= N) continue;
    const int pc = kGated ? (oc / (TN / 2)) * TN + oc % (TN / 2) : oc;
    const float* src = part + r * BN + pc;
    f32x4_t va[kMaxSplitParts], vb[kMaxSplitParts];
#pragma unroll
    for (int p = 0; p < kMaxSplitParts; ++p) {
      if (p < sp) {
        va[p] = *reinterpret_cast<const f32x4_t*>(src + p * (BM * BN));
        if constexpr (kGated) vb[p] = *reinterpret_cast<const f32x4_t*>(src + p * (BM * BN) + TN / 2);
      }
    }
    f32x4_t a = va[0], b = kGated ? vb[0] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 1; p < kMaxSplitParts; ++p) {
      if (p < sp) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          a[c] = a[c] + va[p][c];
          if constexpr (kGated) b[c] = b[c] + vb[p][c];
        }
      }
    }
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = kGated ? silu_mul(a[c], b[c]) : a[c];
    *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row0 + r) * N + col) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

// ---------------------------------------------------------------------------
// Fused expert FFN: FC1 tiles, FC2 tiles and the combine in one persistent
// launch, with device-side readiness counters in place of kernel boundaries
// (the next step the pages' megakernel design points to: FC2 of a block of
// rows may start as soon as that block's FC1 tiles are stored; MegaFlux,
// section 2.1, MegaMoE's tiled FC1/FC2).
//
// The group of workgroups b = x (mod 8) (the workgroups of one XCD) owns, in
// order, its share of the FC1 tiles, then its share of the FC2 tiles, then its
// share of the combine's blocks (512 16-byte vectors of the output, one per
// thread), each share being the tiles the separate launches' XCD-aware
// numbering gives that XCD (so neighbouring tiles meet in one L2); workgroup r
// of the group takes the group's units r, r + W, r + 2W, ... (W workgroups
// per group), with no atomics, and chains consecutive 128-row FC1 tiles as the
// separate launch does.
// An FC2 tile waits until every FC1 tile of its m-block has been stored; a
// combine block waits until every FC2 tile has. No launch can deadlock: a
// workgroup starts its first FC2 tile only after all of its FC1 tiles, which
// never wait, and likewise for FC2 tiles under the combine; the grid is a
// multiple of 8, so every group has workgroups. This needs every workgroup of
// the grid resident at once (the host checks the occupancy before the launch).
// Each wait is bounded: past spin_limit polls the workgroup sets bit 0 of the
// error word and goes on (the results are then wrong, never a hang; the host
// reads the word through moe_fused_status). Producers publish with a device-scope release
// (their stores reach the point of coherence of every XCD's L2); consumers
// take a device-scope acquire before reading.
// sync words: [8] FC2 tiles stored, [kFusedErrorWord] error flags, [11] route
// tiles stored, [12] plan ready, [13] m-block count of the plan, [14] split FC1
// tiles summed, [16 + mb] FC1 tiles of m-block mb stored, then
// [16 + max_mb + i] parts stored of split FC1 tile i and
// [16 + max_mb + kMaxSplitTiles + i] of split FC2 tile i.
//
// Few-tile launches (a decode step: fewer tiles than CUs) split K exactly as
// the separate launches do (the same cut of the same tile list, the parts'
// fp32 accumulators in the same slots of the partial buffer): the workgroup
// that stores a split tile's last part sums the parts in part order and
// applies the epilogue (the separate launches' reduce, the same device code),
// then counts the tile as stored. FC1 and FC2 parts share the partial buffer,
// so an FC2 part starts only once every split FC1 tile has been summed. Tile
// rows (128 for batches with few rows per expert, else 256), FC2 tile width
// and the weight layout (as stored or in stage order) follow the separate
// launches too, so the fused launch's outputs are bitwise theirs.
//
// Route and dispatch as the launch's first phases (front): workgroup b first
// routes tokens b, b + G, ... (a route tile per token: its E logits in the contract order, one
// wave per expert, then its top k and weights, the same device code as the
// small-batch route kernel); the workgroup that stores the last route tile then
// runs the one-workgroup dispatch and tile plan (the same device code as the
// dispatch kernel) and publishes the plan; every other workgroup waits for it
// before the FFN phases. The dispatch places every expert's rows and writes
// the plan in one pass, so readiness per expert would arrive at the same
// moment as the plan. A workgroup whose wait for the plan gives up exits
// without touching the plan (error bit 1): the plan's words may still be
// changing, and the m-block list drives the FFN tiles' addresses. A batch of
// at most kLocalRouteLogits logits (a decode step of a token or two) is
// instead routed and dispatched by every workgroup for itself, which costs a
// few logits per workgroup and no wait at all.
constexpr int kFusedSyncHead = 16;
[[maybe_unused]] constexpr int kSyncRouteDone = 11, kSyncPlanReady = 12, kSyncPlanCount = 13,
              kSyncSplit1Done = 14;
// split tiles of one phase: fewer than the split target (the CU count)
constexpr int kMaxSplitTiles = 1024;
// combine units: 512 consecutive 8-column vectors of the [T][d] output (one per thread)
[[maybe_unused]] constexpr int kCombineVecs = 512;
// batches of at most this many logits (T * E) are routed by every workgroup itself
[[maybe_unused]] constexpr int kLocalRouteLogits = 16;
// elements per lane whose loads a front logit issues at once (a 6144-wide
// logit in two round trips; the registers are free before the FFN phases)
[[maybe_unused]] constexpr int kFrontLoads = 48;

struct FusedFfnArgs {
  GemmArgs fc1, fc2;
  const int32_t* inv_perm;
  const float* topk_w;
  void* out;
  int64_t T, d;
  int k, n_shared;
  int32_t* sync;
  int spin_limit;  // polls of a readiness counter before giving up; < 0: give up at once
  // front phases (route and dispatch in the launch): front = 1; fc1/fc2's
  // n_mblocks then point at sync[kSyncPlanCount]
  int front, E;
  const void* wg;
  const float* bias;
  float* logits;
  int32_t *topk_idx, *counts, *offsets, *perm_out, *inv_perm_out, *n_mblocks_ws;
  float* topk_w_out;
  int4* mblocks_out;
  int64_t max_mb;
  int block_rows;  // rows per m-block of the plan (the tile rows)
};

// Waits (thread 0 polls, the workgroup then meets at a barrier) until *counter
// reaches target; past spin_limit polls it sets `bit` in the error word and
// gives up. Returns whether the target was reached, the same in every thread
// (through `flag`, an LDS word no other part of the workgroup uses meanwhile).
__device__ __forceinline__ bool wait_count(int32_t* counter, int target, int32_t* err, int spin_limit, int* flag,
                                           int bit = 1) {
  if (threadIdx.x == 0) {
    int spins = 0;
    int met = 1;
    while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (spins >= spin_limit) {
        __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        met = 0;
        break;
      }
      // about a microsecond between polls: hundreds of workgroups polling one
      // line at a shorter interval slow the tiles they wait for (measured)
      __builtin_amdgcn_s_sleep(32);
      ++spins;
    }
    *flag = met;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  const bool ok = *flag != 0;
  __syncthreads();  // every thread has read the flag before a later wait rewrites it
  return ok;
}

// Every wave waits until its stores are complete in its XCD's L2, then one
// device-scope release (an L2 write-back) makes all of them visible to the
// other XCDs before the counter moves. A write-back per wave costs about as
// much again as the whole FC1 phase at decode sizes.
__device__ __forceinline__ void publish(int32_t* counter) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are done
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// publish() that also tells whether this workgroup's increment brought the
// counter to `target` (the same answer in every thread).
__device__ __forceinline__ bool publish_last(int32_t* counter, int target, int* flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == target - 1;
  __syncthreads();
  const bool last = *flag != 0;
  __syncthreads();
  return last;
}

// Front phases of a batch of at most kLocalRouteLogits logits: every workgroup
// computes all of them, the top-k and the dispatch itself (the same device
// code, so the same bits), keeping the top-k in LDS, and writes the routing
// arrays and the plan, so no workgroup waits for another; the copies are
// identical, and each workgroup reads back only what it wrote. Workgroup 0
// alone writes the logits.
__device__ __forceinline__ void fused_front_local(const FusedFfnArgs& a, char* lds) {
  float* srow = reinterpret_cast<float*>(lds + 64);          // [T * E <= 16] logits
  int32_t* sidx = reinterpret_cast<int32_t*>(lds + 256);     // [T * k <= 16] top-k experts
  float* sw = reinterpret_cast<float*>(lds + 384);           // [T * k] their weights
  int32_t* wsum = reinterpret_cast<int32_t*>(lds + 512);     // [8]
  float* sel = reinterpret_cast<float*>(lds + 1024);         // [8 waves][64]
  int32_t(*wh)[kMaxExperts] = reinterpret_cast<int32_t(*)[kMaxExperts]>(lds + 4096);  // [8][1024]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nl = static_cast<int>(a.T) * a.E, nk = static_cast<int>(a.T) * a.k;
  for (int p = wv; p < nl; p += 8) {
    const float l = gate_logit_wave<1, kFrontLoads>(a.fc1.A, a.wg, a.bias, p / a.E, p % a.E, a.d);
    if (lane == 0) {
      srow[p] = l;
      if (blockIdx.x == 0) a.logits[p] = l;
    }
  }
  __syncthreads();
  for (int t = wv; t < a.T; t += 8) topk_row(srow + t * a.E, a.E, a.k, sidx + t * a.k, sw + t * a.k, sel + wv * 64);
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < nk) {
    a.topk_idx[threadIdx.x] = sidx[threadIdx.x];
    a.topk_w_out[threadIdx.x] = sw[threadIdx.x];
  }
  dispatch_block<512>(sidx, nk, a.E, a.counts, a.offsets, a.perm_out, a.inv_perm_out, a.block_rows, a.max_mb,
                      a.mblocks_out, a.sync + kSyncPlanCount, wh, wsum);
  // this workgroup's stores are complete, then its L1 is dropped: the FFN
  // phases read the plan, perm and weights back from memory
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (blockIdx.x == 0) *a.n_mblocks_ws = a.sync[kSyncPlanCount];
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Front phases of the fused launch: route tiles, then the dispatch by the
// workgroup that stores the last route tile, then the plan. Returns false if
// this workgroup gave up waiting for the plan (it must then stay away from it).
__device__ __forceinline__ bool fused_front(const FusedFfnArgs& a, char* lds) {
  if (a.T * a.E <= kLocalRouteLogits) {
    fused_front_local(a, lds);
    return true;
  }
  int* s_flag = reinterpret_cast<int*>(lds + 8);
  float* srow = reinterpret_cast<float*>(lds + 64);        // [<= 64] logits of the token
  float* sel = reinterpret_cast<float*>(lds + 512);        // [<= 64] selected logits
  int32_t* wsum = reinterpret_cast<int32_t*>(lds + 1024);  // [8]
  int32_t(*wh)[kMaxExperts] = reinterpret_cast<int32_t(*)[kMaxExperts]>(lds + 2048);  // [8][1024]
  int32_t* err = a.sync + kFusedErrorWord;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // route tile t (one token) is workgroup t % G's, in token order
  for (int64_t t = blockIdx.x; t < a.T; t += gridDim.x) {
    __syncthreads();  // the previous tile's logits are read before they are rewritten
    for (int e = wv; e < a.E; e += 8) {
      const float l = gate_logit_wave<1, kFrontLoads>(a.fc1.A, a.wg, a.bias, t, e, a.d);
      if (lane == 0) {
        srow[e] = l;
        a.logits[t * a.E + e] = l;
      }
    }
    __syncthreads();
    if (wv == 0) topk_row(srow, a.E, a.k, a.topk_idx + t * a.k, a.topk_w_out + t * a.k, sel);
    if (publish_last(a.sync + kSyncRouteDone, static_cast<int>(a.T), s_flag)) {
      // every route tile is stored: this workgroup dispatches
      if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __syncthreads();
      dispatch_block<512>(a.topk_idx, a.T * a.k, a.E, a.counts, a.offsets, a.perm_out, a.inv_perm_out, a.block_rows,
                          a.max_mb, a.mblocks_out, a.sync + kSyncPlanCount, wh, wsum);
      __syncthreads();
      if (threadIdx.x == 0) *a.n_mblocks_ws = a.sync[kSyncPlanCount];  // where a layer call leaves the count
      publish(a.sync + kSyncPlanReady);
    }
  }
  return wait_count(a.sync + kSyncPlanReady, 1, err, a.spin_limit, s_flag, 2);
}


// After storing a split tile's part: whether this workgroup stored the tile's
// last part (then, after an acquire, it sees every part).
__device__ __forceinline__ bool last_part(int32_t* counter, int parts, int* flag) {
  if (!publish_last(counter, parts, flag)) return false;
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  return true;
}

template <int BM, int BN2, int WM2, int WN2, bool kPacked>
__global__ __launch_bounds__(512, 1) void ffn_fused_kernel(FusedFfnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using F1 = DlGemm<kModeFc1, BM, 256, 2, 4, kPacked>;
  using F2 = DlGemm<kModeFc2, BM, BN2, WM2, WN2, kPacked>;
  static_assert(F1::NT == 512 && F2::NT == 512, "both tile forms use 8 waves");
  constexpr int LDS = F1::LDS_BYTES > F2::LDS_BYTES ? F1::LDS_BYTES : F2::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[LDS];
  // an LDS word for the waits, free whenever a wait runs: between tiles, when
  // no loads of a chained tile are in flight (publish() drains them first)
  int* s_flag = reinterpret_cast<int*>(lds + 16);
  if (a.front && !fused_front(a, lds)) return;
  const int nmb = a.fc1.n_mblocks[0];
  const int nbc1 = static_cast<int>((a.fc1.N + 127) / 128);  // FC1 tiles per m-block
  const int nbc2 = static_cast<int>((a.fc2.N + BN2 - 1) / BN2);
  const int64_t nt1 = static_cast<int64_t>(nmb) * nbc1, nt2 = static_cast<int64_t>(nmb) * nbc2;
  const SplitCut c1 = split_cut(a.fc1, nt1), c2 = split_cut(a.fc2, nt2);
  // units: whole tiles, then the parts of the split tiles (DlGemm's virtual tiles)
  const int64_t n1 = c1.full + (nt1 - c1.full) * c1.sp, n2 = c2.full + (nt2 - c2.full) * c2.sp;
  const int64_t nvec = a.d / 8;
  const int64_t nc = (a.T * nvec + kCombineVecs - 1) / kCombineVecs;
  int32_t* fc2_done = a.sync + 8;
  int32_t* err = a.sync + kFusedErrorWord;
  int32_t* done1 = a.sync + kFusedSyncHead;
  int32_t* parts1 = done1 + a.max_mb;
  int32_t* parts2 = parts1 + kMaxSplitTiles;
  // group x = blockIdx.x % 8 owns, in every round of G tiles, tiles
  // x*W .. x*W + W-1 (W = G / 8): its share of n tiles, and its j-th tile
  const int64_t G = gridDim.x, W = G / 8, x = blockIdx.x % 8;
  auto share = [&](int64_t n) { return (n / G) * W + min(max(n % G - x * W, int64_t(0)), W); };
  auto nth = [&](int64_t j) { return (j / W) * G + x * W + j % W; };
  const int64_t s1 = share(n1), s2 = share(n2), sc = share(nc);
  // Workgroup r of group x takes the group's units r, r + W, r + 2W, ...: FC1
  // tiles, then FC2 tiles, then combine units, in one fixed order (no claim
  // atomics). FC1 tiles never wait, and a workgroup finishes all its FC1
  // tiles before its first FC2 tile, which waits only for FC1 tiles; every
  // workgroup is resident (checked on the host), so every wait is met.
  const int64_t r = blockIdx.x / 8;
  int64_t j = r;
  auto post1 = [&](int64_t v, int mb) {
    if (v < c1.full) {
      publish(done1 + mb);
    } else {
      const int64_t t = c1.full + (v - c1.full) / c1.sp;
      if (last_part(parts1 + (t - c1.full), c1.sp, s_flag)) {
        reduce_split_tile<true, BM, 256, 4>(a.fc1, t, c1, nbc1, nmb, threadIdx.x, 512);
        publish(done1 + mb);
        publish(a.sync + kSyncSplit1Done);
      }
    }
  };
  if constexpr (F1::kChain) {
    // 128-row tiles chained as in the separate launch: the last K steps of a
    // tile issue the next tile's first loads when both are whole tiles (then
    // the tile's post only publishes, which touches no LDS)
    if (j < s1) {
      typename F1::Desc cur, nxt;
      F1::describe(a.fc1, nth(j), cur);
      int s0 = 0;
      bool warm = false;
      for (; j < s1; j += W) {
        const int64_t v = nth(j);
        const bool more = j + W < s1;
        if (more) F1::describe(a.fc1, nth(j + W), nxt);
        const bool chain = more && cur.sp == 1 && nxt.sp == 1 && nxt.nk >= F1::NBB;
        F1::run_tile(a.fc1, lds, cur, nxt, chain ? nxt.nk : 0, s0, warm, [&](int mb) { post1(v, mb); });
        s0 = chain ? s0 + cur.nk : 0;
        warm = chain;
        cur = nxt;
      }
    }
  } else {
    for (; j < s1; j += W) {
      const int64_t v = nth(j);
      F1::tile(a.fc1, lds, v, [](int) {}, [&](int mb) { post1(v, mb); });
    }
  }
  for (; j < s1 + s2; j += W) {
    const int64_t v = nth(j - s1);
    const bool part = v >= c2.full;
    F2::tile(a.fc2, lds, v,
             [&](int mb) {
               wait_count(done1 + mb, nbc1, err, a.spin_limit, s_flag);
               // the partial buffer is free once every split FC1 tile is summed
               if (part && c1.sp > 1)
                 wait_count(a.sync + kSyncSplit1Done, static_cast<int>(nt1 - c1.full), err, a.spin_limit, s_flag);
             },
             [&](int) {
               if (!part) {
                 publish(fc2_done);
               } else {
                 const int64_t t = c2.full + (v - c2.full) / c2.sp;
                 if (last_part(parts2 + (t - c2.full), c2.sp, s_flag)) {
                   reduce_split_tile<false, BM, BN2, WN2>(a.fc2, t, c2, nbc2, nmb, threadIdx.x, 512);
                   publish(fc2_done);
                 }
               }
             });
  }
  if (j < s1 + s2 + sc) wait_count(fc2_done, static_cast<int>(nt2), err, a.spin_limit, s_flag);
  for (; j < s1 + s2 + sc; j += W) {
    const int64_t q = nth(j - s1 - s2) * kCombineVecs + threadIdx.x;
    if (q < a.T * nvec)
      combine_vec<1>(a.fc2.C, a.inv_perm, a.topk_w, a.out, a.d, a.k, a.T * a.k, a.n_shared, a.T, q / nvec,
                     q % nvec);
  }
#endif
}

template <bool kGated, int BM, int BN, int WN>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
  constexpr int OC = kGated ? BN / 2 : BN;
  const int nbc = static_cast<int>((g.N + OC - 1) / OC);
  const int nmb = g.n_mblocks[0];
  const int64_t nt = static_cast<int64_t>(nmb) * nbc;
  const SplitCut cut = split_cut(g, nt);
  if (cut.sp <= 1) return;  // the GEMM wrote its outputs itself
  // R workgroups per split tile, each taking every R-th group of columns, so
  // that a few large split tiles (a launch's last round) still spread over
  // the whole grid
  const int64_t ns = nt - cut.full;
  const int64_t R = ns < gridDim.x ? gridDim.x / ns : 1;
  for (int64_t b = blockIdx.x; b < ns * R; b += gridDim.x)
    reduce_split_tile<kGated, BM, BN, WN>(g, cut.full + b / R, cut, nbc, nmb,
                                          threadIdx.x + static_cast<int>(b % R) * blockDim.x,
                                          static_cast<int>(R) * blockDim.x);
}

// Stage order of one expert-weight tensor W [E][N][K] (bf16, N and K multiples
// of 64): the same E x N x K values, as 64-row groups of K/64 blocks of 8 KiB.
// 16-byte unit u = (((e * N/64 + g) * K/64 + kt) * 64 + rr) * 8 + s holds
// elements kt*64 + 8 * (s ^ ((rr / 2) % 8)) .. +7 of row 64g + rr of expert e:
// exactly what the GEMM's loads place in slot s of a stage row whose index is
// rr modulo 64 (the 8-slot XOR swizzle of 128-byte rows), so each K step of a
// column block reads whole 8 KiB blocks.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* w, u32x4_t* out, int64_t units, int64_t K) {
  const int64_t nk = K / 64;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int s = static_cast<int>(u % 8);
    const int rr = static_cast<int>((u / 8) % 64);
    const int64_t kt = (u / 512) % nk;
    const int64_t row = (u / (512 * nk)) * 64 + rr;  // row of the [E*N][K] matrix
    out[u] = *reinterpret_cast<const u32x4_t*>(w + row * K + kt * 64 + 8 * (s ^ ((rr / 2) % 8)));
  }
}

// The same stage order from an expert-weight tensor stored input-major,
// Wt [E][K][N] (the d x f / f x d orientation of the expert matrices): one
// workgroup per 8 KiB block b = (e * N/64 + g) * K/64 + kt of the output. It
// reads the 64 x 64 sub-matrix Wt[e][64kt ..][64g ..] with coalesced 16-byte
// row loads into LDS, then writes the block's 512 units in order, unit
// rr * 8 + s gathering elements 8 * (s ^ ((rr / 2) % 8)) .. +7 of K for output
// row 64g + rr from an LDS column.
__global__ __launch_bounds__(256) void pack_weights_t_kernel(const uint16_t* wt, u32x4_t* out, int64_t N, int64_t K) {
  __shared__ uint16_t t[64][66];  // [k][n]; the 2-element pad spreads a column over the banks
  const int64_t ng = N / 64, nk = K / 64;
  const int64_t b = blockIdx.x;
  const int64_t kt = b % nk, g = (b / nk) % ng, e = b / (nk * ng);
  const uint16_t* src = wt + (e * K + kt * 64) * N + g * 64;
  for (int c = threadIdx.x; c < 512; c += 256) {
    const int r = c / 8, q = c % 8;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(r) * N + q * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[r][q * 8 + 2 * i] = static_cast<uint16_t>(v[i] & 0xffffu);
      t[r][q * 8 + 2 * i + 1] = static_cast<uint16_t>(v[i] >> 16);
    }
  }
  __syncthreads();
  u32x4_t* dst = out + b * 512;
  for (int u = threadIdx.x; u < 512; u += 256) {
    const int sl = u % 8, rr = u / 8;
    const int k0 = 8 * (sl ^ ((rr / 2) % 8));
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = static_cast<uint32_t>(t[k0 + 2 * i][rr]) | (static_cast<uint32_t>(t[k0 + 2 * i + 1][rr]) << 16);
    dst[u] = v;
  }
}

hipError_t launch_pack_weights_t(const void* w1t, const void* w3t, const void* w2t, void* w1p, void* w3p, void* w2p,
                                 int64_t E, int64_t d, int64_t f, hipStream_t s) {
  const void* src[3] = {w1t, w3t, w2t};
  void* dst[3] = {w1p, w3p, w2p};
  // (N, K) of each matrix: W1 and W3 map d inputs to f outputs, W2 f inputs to d outputs
  const int64_t ndim[3] = {f, f, d}, kdim[3] = {d, d, f};
  for (int m = 0; m < 3; ++m) {
    const int64_t blocks = E * (ndim[m] / 64) * (kdim[m] / 64);
    hipLaunchKernelGGL(pack_weights_t_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src[m]), static_cast<u32x4_t*>(dst[m]), ndim[m], kdim[m]);
    if (hipError_t err = hipGetLastError()) return err;
  }
  return hipSuccess;
}

hipError_t launch_pack_weights(const void* w1, const void* w3, const void* w2, void* w1p, void* w3p, void* w2p,
                               int64_t E, int64_t d, int64_t f, hipStream_t s) {
  const int64_t units = E * d * f / 8;  // 16-byte units of one tensor
  const int grid = static_cast<int>(std::min<int64_t>((units + 255) / 256, 65536));
  const void* src[3] = {w1, w3, w2};
  void* dst[3] = {w1p, w3p, w2p};
  const int64_t kdim[3] = {d, d, f};
  for (int t = 0; t < 3; ++t) {
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid), dim3(256), 0, s, static_cast<const uint16_t*>(src[t]),
                       static_cast<u32x4_t*>(dst[t]), units, kdim[t]);
    if (hipError_t err = hipGetLastError()) return err;
  }
  return hipSuccess;
}

// Largest number of K parts per tile: each part keeps at least 8 K steps of
// 64; MOE_SPLIT_K=0 in the environment turns splitting off (=n caps it at n).
static int split_k_parts(int64_t K) {
  int s = static_cast<int>(std::min<int64_t>(kMaxSplitParts, K / (64 * 8)));
  if (const char* env = getenv("MOE_SPLIT_K")) {
    const int v = atoi(env);
    if (v >= 0 && v < s) s = v;
  }
  return s;
}

// Whether a forward launch whose largest plan has nt tiles may split K (K
// dimension K): every tile when even that plan has fewer tiles than CUs, the
// last partial round when it spans two or more rounds. (A launch between the
// two, a batch of a few hundred tokens, does neither, and keeps the smaller
// workspace.)
static bool may_split(int64_t nt, int64_t K) {
  const int64_t cus = device_cu_count();
  return (nt < cus || nt >= 2 * cus) && split_k_parts(K) > 1;
}

size_t splitk_partial_bytes(int dtype, int regime, int64_t max_mb, int64_t d, int64_t f) {
  if (dtype != 1 || regime < 1) return 0;
  const int64_t cus = device_cu_count();
  // FC1 tiles have 128 output columns, FC2 tiles up to 256
  const bool fc1 = may_split(max_mb * ((f + 127) / 128), d);
  const bool fc2 = may_split(max_mb * ((d + 255) / 256), f);
  const int64_t bm = regime_block_rows(regime);
  return fc1 || fc2 ? static_cast<size_t>(cus) * bm * 256 * sizeof(float) : 0;
}

static int persistent_grid(int64_t max_tiles) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 2;
  int64_t g = max_tiles < cap ? max_tiles : cap;
  return static_cast<int>(g < 1 ? 1 : g);
}

int choose_gemm_regime(int64_t T, int k, int E) {
  if (const char* env = getenv("MOE_GEMM_REGIME")) {
    const int r = atoi(env);
    if (r >= 0 && r <= 3) return r;
  }
  // Few rows per expert (decode batches: the expert's weights are read once,
  // by one m-block): 128-row tiles, whose smaller A stages leave LDS for one
  // more weight step in flight. 96 rows on average keeps the busiest experts
  // of balanced routing within one 128-row block. Otherwise 256-row tiles.
  const int64_t n = T * k, active = n < E ? n : E;
  if (active > 0 && (n + active - 1) / active <= 96) return 3;
  return 1;
}

int regime_block_rows(int regime) { return regime == 1 || regime == 2 ? 256 : 128; }

// Large-tile launch: one workgroup of 8 waves per CU (the LDS buffers take up
// to the CU's 160 KB), persistent over the tile list.
template <int kMode, int BM, int BN, int WM, int WN, bool kPacked = false>
static hipError_t launch_big(const GemmArgs& a, int64_t max_mb, int64_t ncols, hipStream_t s) {
  const int64_t cols = mode_gated(kMode) ? BN / 2 : BN;
  const int64_t nb = (ncols + cols - 1) / cols;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(max_mb * nb, device_cu_count())));
  hipLaunchKernelGGL((gemm_dl_kernel<kMode, BM, BN, WM, WN, kPacked>), dim3(grid), dim3(64 * WM * WN), 0, s, a);
  return hipGetLastError();
}

// Forward FC1/FC2 launch, split along K where the partial buffer is there
// (splitk_partial_bytes) and the plan calls for it: a launch with fewer tiles
// than CUs (few rows and few experts: a decode step of a handful of tokens)
// splits every tile, so that its parts run on all CUs; a launch of several
// rounds splits the tiles of its last, partial round, whose CUs would
// otherwise wait for most of a tile (Mixtral-8x22B prefill FC2: 1608 tiles, a
// last round of 72 for 256 CUs). A second kernel sums the parts. FC2 splits
// any partial last round (halving the tiles of the balanced prefill's
// half-full one: FC2 2.75 -> 2.55 ms); FC1 only one cut into three or more
// parts, a round at most a third full (its tiles have fewer K steps, and
// halving the prefill's half-full last round cost 0.5 %, while the DBRX- and
// DeepSeek-shaped FC1 gained 2-3 % from rounds cut into 8).
// Whether a forward launch over up to max_mb m-blocks x nb column blocks
// (tiles of tile_floats fp32 accumulators) splits K, given a partial buffer of
// partial_bytes (0: none), and if so its split fields in a; the plan on the
// device decides which tiles. The fused launch takes the same decision, so its
// tiles split the same way.
static bool fwd_split(GemmArgs& a, int64_t max_mb, int64_t nb, int64_t tile_floats, float* partial,
                      size_t partial_bytes, int tail_min) {
  const int parts = split_k_parts(a.K);
  const int64_t cap = static_cast<int64_t>(partial_bytes / (sizeof(float) * tile_floats));
  if (partial_bytes == 0 || cap < 2 || !may_split(max_mb * nb, a.K)) return false;
  a.partial = partial;
  a.splits = parts;
  a.split_target = static_cast<int>(device_cu_count());
  a.partial_cap = static_cast<int>(cap);
  a.tail_min = tail_min;
  return true;
}

// Tile queues for the 256-row forward launches; MOE_TILE_QUEUES=0 in the
// environment gives every workgroup a fixed share of the tiles instead (the
// same outputs, bit for bit).
static bool tile_queues_on() {
  const char* env = getenv("MOE_TILE_QUEUES");
  return !(env && env[0] == '0');
}

template <int kMode, int BM, int BN, int WM, int WN, bool kPacked = false>
static hipError_t launch_fwd(GemmArgs a, int64_t max_mb, int64_t ncols, float* partial, size_t partial_bytes,
                             bool queues, hipStream_t s) {
  const int64_t cols = mode_gated(kMode) ? BN / 2 : BN;
  const int64_t nb = (ncols + cols - 1) / cols;
  const int64_t cus = device_cu_count();
  // 256-row tiles (not chained) take their tiles from the plan's queues
  static_assert(kMode == kModeFc1 || kMode == kModeFc2, "forward forms");
  if (BM == 256 && queues && tile_queues_on())
    a.tileq = const_cast<int32_t*>(a.n_mblocks) + (kMode == kModeFc1 ? kTileQueueFc1 : kTileQueueFc2);
  if (!fwd_split(a, max_mb, nb, static_cast<int64_t>(BM) * BN, partial, partial_bytes, kMode == kModeFc2 ? 2 : 3))
    return launch_big<kMode, BM, BN, WM, WN, kPacked>(a, max_mb, ncols, s);
  hipLaunchKernelGGL((gemm_dl_kernel<kMode, BM, BN, WM, WN, kPacked>), dim3(static_cast<int>(cus)), dim3(64 * WM * WN), 0, s,
                     a);
  if (hipError_t err = hipGetLastError()) return err;
  hipLaunchKernelGGL((splitk_reduce_kernel<mode_gated(kMode), BM, BN, WN>), dim3(static_cast<int>(2 * cus)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_fc1(int dtype, int regime, const void* x, const int32_t* perm, int k, int64_t T,
                      const void* w1, const void* w3, void* h, const int4* mblocks,
                      const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f,
                      const SharedExperts& sh, float* partial, size_t partial_bytes, bool packed, bool queues,
                      hipStream_t s) {
  GemmArgs a{x, perm, k, T, w1, w3, h, mblocks, n_mblocks, d, f,
             T * k, sh.w1, sh.w3, sh.n > 0 ? sh.E_routed : INT32_MAX};
  // packed: w1, w3 in stage order (pack_weights_kernel), read by the large-tile
  // kernels only
  if (dtype == 1 && packed)
    return regime == 3 ? launch_fwd<kModeFc1, 128, 256, 2, 4, true>(a, max_mb, f, partial, partial_bytes, queues, s)
                       : launch_fwd<kModeFc1, 256, 256, 2, 4, true>(a, max_mb, f, partial, partial_bytes, queues, s);
  if (dtype == 1 && regime == 3)
    return launch_fwd<kModeFc1, 128, 256, 2, 4>(a, max_mb, f, partial, partial_bytes, queues, s);
  if (dtype == 1 && regime >= 1)
    return launch_fwd<kModeFc1, 256, 256, 2, 4>(a, max_mb, f, partial, partial_bytes, queues, s);
  const int grid = persistent_grid(max_mb * (f / (kBNW / 2)));
  if (dtype == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<1, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<0, true>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// Few m-blocks (decode-sized batches, weight streaming): 256-column FC2 tiles
// can leave CUs idle (Mixtral-8x22B decode: 8 x 24 tiles for 256 CUs);
// 192-column tiles (8 x 32 there, one per CU) are taken when their rounds of
// tiles cost less for the expected number of m-blocks. Regime 2 keeps 256.
static bool fc2_narrow(int regime, int64_t est_mb, int64_t d) {
  const int64_t cus = device_cu_count();
  if (regime == 2 || est_mb * ((d + 255) / 256) >= 2 * cus) return false;
  const int64_t t256 = (est_mb * ((d + 255) / 256) + cus - 1) / cus * 256;
  const int64_t t192 = (est_mb * ((d + 191) / 192) + cus - 1) / cus * 192;
  return t192 < t256;
}

hipError_t launch_fc2(int dtype, int regime, const void* h, const void* w2, void* y, const int4* mblocks,
                      const int32_t* n_mblocks, int64_t max_mb, int64_t est_mb, int64_t d, int64_t f,
                      const SharedExperts& sh, float* partial, size_t partial_bytes, bool packed, bool queues,
                      hipStream_t s) {
  GemmArgs a{h, nullptr, 1, 0, w2, nullptr, y, mblocks, n_mblocks, f, d,
             0, sh.w2, nullptr, sh.n > 0 ? sh.E_routed : INT32_MAX};
  if (dtype == 1 && regime >= 1) {
    const bool narrow = fc2_narrow(regime, est_mb, d);
    if (packed) {  // W2 in stage order (pack_weights_kernel)
      if (regime == 3)
        return narrow ? launch_fwd<kModeFc2, 128, 192, 2, 4, true>(a, max_mb, d, partial, partial_bytes, queues, s)
                      : launch_fwd<kModeFc2, 128, 256, 2, 4, true>(a, max_mb, d, partial, partial_bytes, queues, s);
      return narrow ? launch_fwd<kModeFc2, 256, 192, 4, 2, true>(a, max_mb, d, partial, partial_bytes, queues, s)
                    : launch_fwd<kModeFc2, 256, 256, 2, 4, true>(a, max_mb, d, partial, partial_bytes, queues, s);
    }
    if (regime == 3)
      return narrow ? launch_fwd<kModeFc2, 128, 192, 2, 4>(a, max_mb, d, partial, partial_bytes, queues, s)
                    : launch_fwd<kModeFc2, 128, 256, 2, 4>(a, max_mb, d, partial, partial_bytes, queues, s);
    return narrow ? launch_fwd<kModeFc2, 256, 192, 4, 2>(a, max_mb, d, partial, partial_bytes, queues, s)
                  : launch_fwd<kModeFc2, 256, 256, 2, 4>(a, max_mb, d, partial, partial_bytes, queues, s);
  }
  const int grid = persistent_grid(max_mb * ((d + kBNW - 1) / kBNW));
  if (dtype == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<1, false>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<0, false>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------- backward GEMMs (bf16, 256 x 256 tiles) ----------------

hipError_t launch_fc1_gu(const void* x, const int32_t* perm, int k, int64_t T, const void* w1, const void* w3,
                         void* gu, const int4* mblocks, const int32_t* n_mblocks, int64_t max_mb, int64_t d,
                         int64_t f, hipStream_t s, void* h) {
  GemmArgs a{x, perm, k, T, w1, w3, gu, mblocks, n_mblocks, d, f, T * k, nullptr, nullptr, INT32_MAX};
  a.C2 = h;
  return launch_big<kModeFc1GU, 256, 256, 2, 4>(a, max_mb, f, s);
}

hipError_t launch_bwd_q(const void* dout, const int32_t* perm, int k, int64_t T, const void* w2, float* q,
                        const int4* mblocks, const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f,
                        hipStream_t s) {
  GemmArgs a{dout, perm, k, T, w2, nullptr, q, mblocks, n_mblocks, d, f, T * k, nullptr, nullptr, INT32_MAX};
  return launch_big<kModeBwdQ, 256, 256, 2, 4>(a, max_mb, f, s);
}

hipError_t launch_bwd_dx(const void* dgu, const void* w1, const void* w3, float* dxs, const int4* mblocks,
                         const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f, hipStream_t s) {
  // two passes over the dg|du rows: dxs = dg W1, then dxs += du W3
  GemmArgs a{dgu, nullptr, 1, 0, w1, nullptr, dxs, mblocks, n_mblocks, f, d, 0, nullptr, nullptr, INT32_MAX};
  a.a_pitch = 2 * f;
  if (hipError_t err = launch_big<kModeBwdDx, 256, 256, 2, 4>(a, max_mb, d, s)) return err;
  a.B0 = w3;
  a.a_col0 = f;
  a.accumulate = 1;
  return launch_big<kModeBwdDx, 256, 256, 2, 4>(a, max_mb, d, s);
}

hipError_t launch_wgrad(const void* at, const void* bt, void* c, void* c2, const int32_t* kofs, int64_t pitch,
                        int E, int64_t M, int64_t N, int64_t split, hipStream_t s, bool out_bf16) {
  GemmArgs a{at, nullptr, 1, 0, bt, nullptr, c, nullptr, nullptr, 0, N, 0, nullptr, nullptr, INT32_MAX,
             c2, kofs, pitch, M, split, E};
  a.out_bf16 = out_bf16 ? 1 : 0;
  const int64_t tiles = static_cast<int64_t>(E) * (M / 256) * (N / 256);
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(tiles, device_cu_count())));
  hipLaunchKernelGGL((gemm_dl_kernel<kModeWgrad, 256, 256, 2, 4>), dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

size_t fused_sync_words(int64_t max_mb) {
  return static_cast<size_t>(kFusedSyncHead + max_mb + 2 * kMaxSplitTiles);
}

// One form of the fused kernel: launched (per_cu null) or its occupancy queried.
template <int BM, int BN2, int WM2, int WN2, bool kPacked>
static hipError_t fused_form(const FusedFfnArgs* a, int grid, hipStream_t s, int* per_cu) {
  if (per_cu)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, ffn_fused_kernel<BM, BN2, WM2, WN2, kPacked>, 512, 0);
  hipLaunchKernelGGL((ffn_fused_kernel<BM, BN2, WM2, WN2, kPacked>), dim3(grid), dim3(512), 0, s, *a);
  return hipGetLastError();
}

template <bool kPacked>
static hipError_t fused_form_rows(bool rows128, bool narrow, const FusedFfnArgs* a, int grid, hipStream_t s,
                                  int* per_cu) {
  // the separate launches' tile forms (launch_fc1, launch_fc2)
  if (rows128)
    return narrow ? fused_form<128, 192, 2, 4, kPacked>(a, grid, s, per_cu)
                  : fused_form<128, 256, 2, 4, kPacked>(a, grid, s, per_cu);
  return narrow ? fused_form<256, 192, 4, 2, kPacked>(a, grid, s, per_cu)
                : fused_form<256, 256, 2, 4, kPacked>(a, grid, s, per_cu);
}

// Tile form, split fields and grid of a fused launch (args a with fc1/fc2
// set): the separate launches' choices for the same regime, a multiple of 8
// workgroups (every tile group must have workgroups), at most one per CU, all
// CUs when a phase splits.
struct FusedShape {
  bool rows128, narrow;
  int grid;
};
static FusedShape fused_shape(FusedFfnArgs& a, int regime, int64_t max_mb, int64_t est_mb, int64_t d, int64_t f,
                              float* partial, size_t partial_bytes) {
  FusedShape sh{};
  sh.rows128 = regime == 3;
  sh.narrow = fc2_narrow(regime, est_mb, d);
  const int64_t bm = sh.rows128 ? 128 : 256, bn2 = sh.narrow ? 192 : 256;
  const bool sp1 = fwd_split(a.fc1, max_mb, (f + 127) / 128, bm * 256, partial, partial_bytes, 3);
  const bool sp2 = fwd_split(a.fc2, max_mb, (d + bn2 - 1) / bn2, bm * bn2, partial, partial_bytes, 2);
  const int64_t cus = device_cu_count();
  const int64_t g = (sp1 || sp2 ? cus : std::min<int64_t>(max_mb * ((f + 127) / 128), cus)) / 8 * 8;
  sh.grid = static_cast<int>(g < 8 ? 8 : g);
  return sh;
}

bool ffn_fused_coresident(int regime, bool packed, int64_t max_mb, int64_t est_mb, int64_t d, int64_t f,
                          size_t partial_bytes) {
  FusedFfnArgs a{};
  a.fc1.K = d;
  a.fc2.K = f;
  // (the buffer's size decides whether a phase splits; its address is not needed here)
  const FusedShape sh = fused_shape(a, regime, max_mb, est_mb, d, f, nullptr, partial_bytes);
  int per_cu = 0;
  const hipError_t e = packed ? fused_form_rows<true>(sh.rows128, sh.narrow, &a, sh.grid, nullptr, &per_cu)
                              : fused_form_rows<false>(sh.rows128, sh.narrow, &a, sh.grid, nullptr, &per_cu);
  return e == hipSuccess && static_cast<int64_t>(per_cu) * device_cu_count() >= sh.grid;
}

bool fused_front_ok(int64_t T, int E, int k) {
  if (const char* env = getenv("MOE_FUSED_FRONT"))
    if (env[0] == '0') return false;
  return T >= 1 && E <= 64 && T * k <= kFusedMaxAssign;
}

// (Route, dispatch,) FC1, FC2 and combine in one launch (bf16). The sync words
// must be zero on entry.
hipError_t launch_ffn_fused(int regime, bool packed, const void* x, const int32_t* perm, int k, int64_t T,
                            const void* w1, const void* w3, const void* w2, void* h, void* y, int4* mblocks,
                            int32_t* n_mblocks, int64_t max_mb, int64_t est_mb, int64_t d, int64_t f,
                            const int32_t* inv_perm, const float* topk_w, void* out, int32_t* sync,
                            const SharedExperts& sh, float* partial, size_t partial_bytes, int spin_limit,
                            const FusedFront& front, hipStream_t s) {
  FusedFfnArgs a{};
  a.fc1 = GemmArgs{x, perm, k, T, w1, w3, h, mblocks, n_mblocks, d, f, T * k, sh.w1, sh.w3,
                   sh.n > 0 ? sh.E_routed : INT32_MAX};
  a.fc2 = GemmArgs{h, nullptr, 1, 0, w2, nullptr, y, mblocks, n_mblocks, f, d, 0, sh.w2, nullptr,
                   sh.n > 0 ? sh.E_routed : INT32_MAX};
  a.inv_perm = inv_perm;
  a.topk_w = topk_w;
  a.out = out;
  a.T = T;
  a.d = d;
  a.k = k;
  a.n_shared = sh.n;
  a.sync = sync;
  a.spin_limit = spin_limit;
  a.max_mb = max_mb;
  a.block_rows = regime_block_rows(regime);
  if (front.on) {
    // the launch routes and dispatches first; its FFN phases read the plan's
    // count from the sync words
    a.front = 1;
    a.E = front.E;
    a.wg = front.wg;
    a.bias = front.bias;
    a.logits = front.logits;
    a.topk_idx = front.topk_idx;
    a.topk_w_out = front.topk_w;
    a.counts = front.counts;
    a.offsets = front.offsets;
    a.perm_out = front.perm;
    a.inv_perm_out = front.inv_perm;
    a.mblocks_out = mblocks;
    a.n_mblocks_ws = n_mblocks;
    a.fc1.n_mblocks = a.fc2.n_mblocks = sync + kSyncPlanCount;
  }
  const FusedShape fs = fused_shape(a, regime, max_mb, est_mb, d, f, partial, partial_bytes);
  return packed ? fused_form_rows<true>(fs.rows128, fs.narrow, &a, fs.grid, s, nullptr)
                : fused_form_rows<false>(fs.rows128, fs.narrow, &a, fs.grid, s, nullptr);
}

}  // namespace moe
