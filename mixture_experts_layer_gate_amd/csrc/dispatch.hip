// Dispatch: per-expert histogram, exclusive scan and the stable permutation.
//
// Steps 2 and 4 of the routing pipeline (count tokens per expert, scatter
// them into per-expert buffers; MegaScale-Infer, "Fused Kernels"), with the
// order inside each expert by token, then top-k slot (MegaFlux, appendix A.2).
// Here the scatter produces index maps (perm: sorted position -> assignment,
// inv_perm: assignment -> sorted position); the grouped GEMM gathers rows
// through them instead of copying tokens.
//
// Determinism: LDS atomics only count. Positions come from wave ballots (rank
// among same-expert lanes with a lower lane id) plus per-wave and per-chunk
// prefix counts, so the result never depends on atomic ordering.
#include "common.h"
#include "dispatch_block.h"
#include "kernels.h"

namespace moe {

constexpr int kDispThreads = 256;

void dispatch_chunking(int64_t n, int* chunk, int* n_chunks) {
  // chunk = 256 * rounds, so that there are at most 1024 chunks
  int64_t rounds = (n + int64_t(kDispThreads) * 1024 - 1) / (int64_t(kDispThreads) * 1024);
  if (rounds < 1) rounds = 1;
  *chunk = static_cast<int>(rounds * kDispThreads);
  *n_chunks = static_cast<int>((n + *chunk - 1) / *chunk);
  if (*n_chunks < 1) *n_chunks = 1;
}


__global__ __launch_bounds__(kDispThreads) void hist_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                             int E, int chunk,
                                                             int32_t* __restrict__ block_hist) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kDispThreads) h[e] = 0;
  __syncthreads();
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * chunk;
  for (int i = threadIdx.x; i < chunk; i += kDispThreads) {
    const int64_t a = a0 + i;
    if (a < n) atomicAdd(&h[clamp_expert(idx[a], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kDispThreads)
    block_hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

// One block: column prefix over chunks (per expert), counts, exclusive scan over
// experts, then block_hist[b][e] becomes the first sorted position of chunk b's
// assignments to expert e.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ block_hist, int n_chunks,
                                                    int E, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  constexpr int kBatch = 16;  // chunk counts loaded together, then rewritten
  int32_t run = 0;
  if (e < E) {
    for (int b0 = 0; b0 < n_chunks; b0 += kBatch) {
      int32_t c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        c[j] = b0 + j < n_chunks ? block_hist[static_cast<int64_t>(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (b0 + j < n_chunks) {
          block_hist[static_cast<int64_t>(b0 + j) * E + e] = run;
          run += c[j];
        }
    }
    counts[e] = run;
  }
  // exclusive scan of run over e (1024 threads = 16 waves)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int32_t incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  const int32_t excl = before + incl - run;
  if (e < E) {
    tot[e] = excl;
    offsets[e] = excl;
  }
  if (e == E - 1) offsets[E] = excl + run;
  __syncthreads();
  if (e < E)
    for (int b = 0; b < n_chunks; ++b) block_hist[static_cast<int64_t>(b) * E + e] += tot[e];
}

__global__ __launch_bounds__(kDispThreads) void scatter_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                                int E, int chunk,
                                                                const int32_t* __restrict__ block_base,
                                                                int32_t* __restrict__ perm,
                                                                int32_t* __restrict__ inv_perm) {
  constexpr int kWaves = kDispThreads / kWave;
  __shared__ int32_t base[kMaxExperts];
  __shared__ int32_t wcnt[kWaves][kMaxExperts];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += kDispThreads)
    base[e] = block_base[static_cast<int64_t>(blockIdx.x) * E + e];
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * chunk;
  for (int r0 = 0; r0 < chunk; r0 += kDispThreads) {
    for (int i = threadIdx.x; i < kWaves * E; i += kDispThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int64_t a = a0 + r0 + threadIdx.x;
    const bool valid = a < n;
    const int e = valid ? clamp_expert(idx[a], E) : 0;
    // lanes of this wave holding the same expert
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int32_t pos = base[e] + rank;
      for (int w = 0; w < wv; ++w) pos += wcnt[w][e];
      // positions are in [0, n) by construction; the guard keeps a bad count
      // from ever turning into a write outside perm
      if (pos >= 0 && pos < n) perm[pos] = static_cast<int32_t>(a);
      inv_perm[a] = pos;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += kDispThreads) {
      int32_t add = 0;
      for (int w = 0; w < kWaves; ++w) add += wcnt[w][x];
      base[x] += add;
    }
    __syncthreads();
  }
}

// Tile group of an expert's i-th m-block (of nb, the first at list index
// start): runs of up to kTileGroup consecutive m-blocks of one expert, packed
// as (index of the group's first m-block) << 4 | (group size). The grouped
// GEMM walks a group's tiles m-block-fastest, so the CUs that run them at the
// same time share weight and activation panels.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;

__global__ __launch_bounds__(kFusedThreads) void dispatch_fused_kernel(
    const int32_t* __restrict__ idx, int64_t n, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int block_rows, int64_t max_mb, int4* __restrict__ mblocks, int32_t* __restrict__ n_mblocks) {
  __shared__ int32_t wh[kFusedWaves][kMaxExperts];  // per-wave counts, then per-wave running positions
  __shared__ int32_t wsum[kFusedWaves];
  dispatch_block<kFusedThreads, true>(idx, n, E, counts, offsets, perm, inv_perm, block_rows, max_mb, mblocks, n_mblocks,
                                wh, wsum);
}

hipError_t launch_dispatch_fused(const int32_t* idx, int64_t n, int E, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* inv_perm, int block_rows, int64_t max_mb,
                                 int4* mblocks, int32_t* n_mblocks, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_fused_kernel, dim3(1), dim3(kFusedThreads), 0, s, idx, n, E, counts, offsets, perm,
                     inv_perm, block_rows, max_mb, mblocks, n_mblocks);
  return hipGetLastError();
}

hipError_t launch_hist(const int32_t* idx, int64_t n, int E, int chunk, int n_chunks,
                       int32_t* block_hist, hipStream_t s) {
  hipLaunchKernelGGL(hist_kernel, dim3(n_chunks), dim3(kDispThreads), 0, s, idx, n, E, chunk, block_hist);
  return hipGetLastError();
}

hipError_t launch_scan(int32_t* block_hist, int n_chunks, int E, int32_t* counts, int32_t* offsets,
                       hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, block_hist, n_chunks, E, counts, offsets);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, int64_t n, int E, int chunk, int n_chunks,
                          const int32_t* block_base, int32_t* perm, int32_t* inv_perm, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(n_chunks), dim3(kDispThreads), 0, s, idx, n, E, chunk,
                     block_base, perm, inv_perm);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile plan: every expert's sorted rows cut into m-blocks of at most
// block_rows rows, only the last one partial (MegaFlux, section 3.1).
// m-blocks are listed in expert order: (expert, first sorted row, rows, 0).
int64_t max_mblocks(int64_t n_assign, int E) {
  const int64_t active = n_assign < E ? n_assign : E;
  return (n_assign + kBlockRows - 1) / kBlockRows + active;
}

// counts/offsets are clamped into [0, n_assign] and the list into max_mb
// entries, so inconsistent caller-provided counts cannot send the GEMM out of
// bounds (they give unspecified rows instead).
// Shared experts (n_shared > 0) follow the E routed ones as experts E .. E+n_shared-1,
// each with T rows starting at sorted row n_assign + s*T.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int64_t n_assign, int64_t max_mb, int block_rows,
                                                    int4* __restrict__ mblocks,
                                                    int32_t* __restrict__ n_mblocks, int n_shared, int64_t T) {
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  int64_t row0 = 0;
  int c = 0;
  if (e < E) {
    row0 = min(max(static_cast<int64_t>(offsets[e]), int64_t(0)), n_assign);
    c = static_cast<int>(min(max(static_cast<int64_t>(counts[e]), int64_t(0)), n_assign - row0));
  } else if (e < E + n_shared) {
    row0 = n_assign + static_cast<int64_t>(e - E) * T;
    c = static_cast<int>(T);
  }
  const int nb = (c + block_rows - 1) / block_rows;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = nb;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  const int start = before + incl - nb;
  if (e < E + n_shared) {
    for (int i = 0; i < nb && start + i < max_mb; ++i) {
      const int r = min(block_rows, c - i * block_rows);
      mblocks[start + i] = make_int4(e, static_cast<int>(row0) + i * block_rows, r, tile_group(start, i, nb));
    }
  }
  const int multi = __syncthreads_or(e < E + n_shared && nb > 1);
  if (e == 1023) {
    n_mblocks[0] = static_cast<int32_t>(min(static_cast<int64_t>(before + incl), max_mb));
    n_mblocks[kPlanMulti] = multi ? 1 : 0;
    for (int i = 0; i < 2 * kTileQueueWords; ++i) n_mblocks[kTileQueueFc1 + i * kTileQueueStride] = 0;
  }
}

hipError_t launch_plan(const int32_t* counts, const int32_t* offsets, int E, int64_t n_assign,
                       int64_t max_mb, int block_rows, int4* mblocks, int32_t* n_mblocks, hipStream_t s,
                       int n_shared, int64_t T) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, E, n_assign, max_mb, block_rows,
                     mblocks, n_mblocks, n_shared, T);
  return hipGetLastError();
}

}  // namespace moe
