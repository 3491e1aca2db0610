// The one-workgroup dispatch as a device function, shared by its own kernel
// (1024 threads) and the fused layer launch (512 threads), so that both give
// the same counts, offsets, permutation and tile plan.
//
// Steps 2 and 4 of the routing pipeline (count tokens per expert, scatter
// them into per-expert order; MegaScale-Infer, "Fused Kernels"), with the order
// inside each expert by token, then top-k slot (MegaFlux, appendix A.2), and
// the tile plan of at most one partial block per expert (MegaFlux, section 3.1).
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxExperts = 1024;

__device__ __forceinline__ int clamp_expert(int e, int E) { return min(max(e, 0), E - 1); }

__device__ __forceinline__ int tile_group(int start, int i, int nb) {
  const int g0 = (i / kTileGroup) * kTileGroup;
  return ((start + g0) << 4) | min(kTileGroup, nb - g0);
}

// ---------------------------------------------------------------------------
// Single-workgroup dispatch for small batches (n <= kFusedMaxAssign): the
// histogram, the exclusive scan, the stable scatter and (optionally) the tile
// plan in one launch. Each of the NT / 64 waves owns one contiguous slice of
// the assignments (slices in assignment order): pass 1 counts its slice into a
// wave-private histogram; one scan gives every (wave, expert) pair its first
// sorted position; pass 2 walks the slice in order, 64 at a time, ranking
// same-expert lanes with ballots and advancing the wave's private running
// positions -- no barriers inside the pass. Same result as the multi-kernel
// path, whatever NT. Thread e scans expert e, so E <= NT; wh [NT/64][1024] and
// wsum [NT/64] are LDS arrays of the caller; every thread of the workgroup
// calls it. kQueues: the count heads a plan piece of the workspace, whose
// multi-block flag is written and tile-queue counters zeroed with it (not
// where the fused launch keeps the count among its readiness counters).

template <int NT, bool kQueues = false>
__device__ __forceinline__ void dispatch_block(const int32_t* __restrict__ idx, int64_t n, int E,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                               int block_rows, int64_t max_mb, int4* __restrict__ mblocks,
                                               int32_t* __restrict__ n_mblocks, int32_t (*wh)[kMaxExperts],
                                               int32_t* wsum) {
  constexpr int kFusedThreads = NT, kFusedWaves = NT / kWave;
  static_assert(NT % kWave == 0 && NT <= 1024, "whole waves");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t slice = (n + kFusedWaves - 1) / kFusedWaves;
  const int64_t a_begin = static_cast<int64_t>(wv) * slice;
  const int64_t a_end = min(n, a_begin + slice);
  for (int i = tid; i < kFusedWaves * E; i += kFusedThreads) wh[i / E][i % E] = 0;
  __syncthreads();
  for (int64_t a = a_begin + lane; a < a_end; a += kWave) atomicAdd(&wh[wv][clamp_expert(idx[a], E)], 1);
  __syncthreads();
  // thread e: total count of expert e and the per-wave prefix (in slice order)
  int c = 0;
  if (tid < E)
    for (int w = 0; w < kFusedWaves; ++w) c += wh[w][tid];
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  const int excl = before + incl - c;
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = excl;
    int run = excl;
    for (int w = 0; w < kFusedWaves; ++w) {
      const int cw = wh[w][tid];
      wh[w][tid] = run;
      run += cw;
    }
  }
  if (tid == E - 1) offsets[E] = excl + c;
  // tile plan from the same counts
  if (mblocks) {
    const int nb = (c + block_rows - 1) / block_rows;
    int bi = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(bi, off);
      if (lane >= off) bi += o;
    }
    __syncthreads();
    if (lane == 63) wsum[wv] = bi;
    __syncthreads();
    int bbefore = 0;
    for (int w = 0; w < wv; ++w) bbefore += wsum[w];
    const int start = bbefore + bi - nb;
    if (tid < E)
      for (int i = 0; i < nb && start + i < max_mb; ++i)
        mblocks[start + i] = make_int4(tid, excl + i * block_rows, min(block_rows, c - i * block_rows),
                                       tile_group(start, i, nb));
    if constexpr (kQueues) {
      const int multi = __syncthreads_or(tid < E && nb > 1);
      if (tid == kFusedThreads - 1) {
        n_mblocks[0] = static_cast<int32_t>(min(static_cast<int64_t>(bbefore + bi), max_mb));
        n_mblocks[kPlanMulti] = multi ? 1 : 0;
        for (int i = 0; i < 2 * kTileQueueWords; ++i) n_mblocks[kTileQueueFc1 + i * kTileQueueStride] = 0;
      }
    } else if (tid == kFusedThreads - 1) {
      n_mblocks[0] = static_cast<int32_t>(min(static_cast<int64_t>(bbefore + bi), max_mb));
    }
  }
  __syncthreads();
  // pass 2: stable scatter of this wave's slice, 64 assignments at a time
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t r0 = a_begin; r0 < a_end; r0 += kWave) {
    const int64_t a = r0 + lane;
    const bool valid = a < a_end;
    const int e = valid ? clamp_expert(idx[a], E) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(peers & lt_mask);
    int32_t pos = 0;
    if (valid) {
      pos = wh[wv][e] + rank;
      if (pos >= 0 && pos < n) perm[pos] = static_cast<int32_t>(a);
      inv_perm[a] = pos;
    }
    // every lane has read its base before the group leaders advance them
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) wh[wv][e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}


}  // namespace moe
