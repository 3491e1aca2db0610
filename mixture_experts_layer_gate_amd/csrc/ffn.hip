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
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kBM = 128;     // rows per tile (== kBlockRows)
constexpr int kBNW = 128;    // weight rows per tile
constexpr int kBK = 64;      // K per step
constexpr int kThreads = 256;
static_assert(kBM == kBlockRows, "tile rows must match the plan's block rows");

struct GemmArgs {
  const void* A;          // FC1: x [T][K]; FC2: h [T*k][K]
  const int32_t* perm;    // FC1: sorted row -> assignment
  int ktop;               // FC1: token = perm[p] / ktop
  int64_t T;              // FC1: token count (clamp)
  const void* B0;         // FC1: W1 [E][N][K]; FC2: W2 [E][N][K]
  const void* B1;         // FC1: W3 [E][N][K]
  void* C;                // FC1: h [T*k][N]; FC2: y [T*k][N]
  const int4* mblocks;    // (expert, first sorted row, rows, 0)
  const int32_t* n_mblocks;
  int64_t K, N;
};

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
      if constexpr (kGated) {
        int64_t tok = g.perm[rr] / g.ktop;
        tok = tok < 0 ? 0 : (tok >= g.T ? g.T - 1 : tok);
        arow = tok;
      } else {
        arow = rr;
      }
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
        base = static_cast<const char*>(r < kBNW / 2 ? g.B0 : g.B1);
        n = static_cast<int64_t>(nb) * (kBNW / 2) + (r % (kBNW / 2));
      } else {
        base = static_cast<const char*>(g.B0);
        n = static_cast<int64_t>(nb) * kBNW + r;
        if (n >= N) n = N - 1;
      }
      bptr_[i] = base + ((static_cast<int64_t>(e) * N + n) * K) * EB + bcol[i] * 16;
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

static int persistent_grid(int64_t max_tiles) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 2;
  int64_t g = max_tiles < cap ? max_tiles : cap;
  return static_cast<int>(g < 1 ? 1 : g);
}

hipError_t launch_fc1(int dtype, const void* x, const int32_t* perm, int k, int64_t T,
                      const void* w1, const void* w3, void* h, const int4* mblocks,
                      const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f, hipStream_t s) {
  GemmArgs a{x, perm, k, T, w1, w3, h, mblocks, n_mblocks, d, f};
  const int grid = persistent_grid(max_mb * (f / (kBNW / 2)));
  if (dtype == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<1, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<0, true>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fc2(int dtype, const void* h, const void* w2, void* y, const int4* mblocks,
                      const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f, hipStream_t s) {
  GemmArgs a{h, nullptr, 1, 0, w2, nullptr, y, mblocks, n_mblocks, f, d};
  const int grid = persistent_grid(max_mb * ((d + kBNW - 1) / kBNW));
  if (dtype == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<1, false>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<0, false>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
