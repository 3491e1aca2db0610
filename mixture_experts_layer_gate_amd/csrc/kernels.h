// Host-side launchers of the MoE-layer kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Smallest rows per m-block of the grouped GEMM (tile-aligned token blocks);
// the large-tile regimes use 256.
constexpr int kBlockRows = 128;
// Largest tile group (m-blocks of one expert walked together by the GEMM).
constexpr int kTileGroup = 8;

// Gate logits l[t][e] in the fixed fp32 order. Requires d % 8 == 0.
// Whether launch_gate_logits runs the gate of a T x d x E batch on the fp32
// matrix cores (gate_mfma_kernel) rather than the vector ALUs.
bool gate_uses_mfma(int dtype, int64_t T, int64_t d, int E);
hipError_t launch_gate_logits(int dtype, const void* x, const void* wg, const float* bias,
                              float* logits, int64_t T, int64_t d, int E, hipStream_t s);
// Top-k selection + renormalised softmax weights from logits.
hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                       hipStream_t s);
// Gate + top-k in one launch for small batches (E <= 16, T * E <= 4096, no
// forced gate tiling): the same logits, bit for bit, and the same selection.
bool route_small_ok(int64_t T, int E);
hipError_t launch_route_small(int dtype, const void* x, const void* wg, const float* bias, float* logits, int64_t T,
                              int64_t d, int E, int k, int32_t* idx, float* w, hipStream_t s);

// Dispatch. n = T*k assignments, cut into n_chunks chunks of `chunk` assignments.
void dispatch_chunking(int64_t n, int* chunk, int* n_chunks);
hipError_t launch_hist(const int32_t* idx, int64_t n, int E, int chunk, int n_chunks,
                       int32_t* block_hist, hipStream_t s);
hipError_t launch_scan(int32_t* block_hist, int n_chunks, int E, int32_t* counts, int32_t* offsets,
                       hipStream_t s);
hipError_t launch_scatter(const int32_t* idx, int64_t n, int E, int chunk, int n_chunks,
                          const int32_t* block_base, int32_t* perm, int32_t* inv_perm, hipStream_t s);

// Single-workgroup dispatch (+ tile plan when mblocks != nullptr) for
// n <= kFusedMaxAssign assignments.
constexpr int64_t kFusedMaxAssign = 65536;
hipError_t launch_dispatch_fused(const int32_t* idx, int64_t n, int E, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* inv_perm, int block_rows, int64_t max_mb,
                                 int4* mblocks, int32_t* n_mblocks, hipStream_t s);

// Tile plan: m-blocks (expert, first sorted row, rows, 0) of at most block_rows rows.
// The m-block count n_mblocks[0] heads a workspace piece of kPlanWords
// words that also holds, in word kPlanMulti, whether some expert's rows span
// more than one m-block, and the tile queues of the FC1 and FC2 launches
// reading the plan: 8 counters each (one per XCD), kTileQueueStride words
// apart so that no two share a cache line, at kTileQueueFc1 and kTileQueueFc2
// + q * kTileQueueStride; the kernel that writes the count writes the flag
// and zeroes the counters.
constexpr int kPlanMulti = 1;
constexpr int kTileQueueStride = 64, kTileQueueWords = 8;
constexpr int kTileQueueFc1 = kTileQueueStride, kTileQueueFc2 = kTileQueueFc1 + kTileQueueWords * kTileQueueStride;
constexpr int kPlanWords = kTileQueueFc2 + kTileQueueWords * kTileQueueStride;
int64_t max_mblocks(int64_t n_assign, int E);
// With n_shared > 0, shared experts E .. E+n_shared-1 of T rows each follow the
// routed rows (E + n_shared <= 1024).
hipError_t launch_plan(const int32_t* counts, const int32_t* offsets, int E, int64_t n_assign,
                       int64_t max_mb, int block_rows, int4* mblocks, int32_t* n_mblocks, hipStream_t s,
                       int n_shared = 0, int64_t T = 0);

// Grouped GEMMs over the m-block list. regime 0: 128 x 128 tiles, register-
// staged, two workgroups per CU (the fp32 path); 1: 256-row tiles fed by
// buffer loads into LDS, 8 waves, one workgroup per CU (bf16), FC1 256 weight
// rows wide, FC2 256 or, when few m-blocks would leave CUs idle, 192
// columns; 2: as 1 with FC2 always 256 columns; 3: as 1 with 128-row tiles
// and m-blocks (few rows per expert: one more weight step in flight).
// MOE_GEMM_REGIME overrides the choice.
// Shared (always-active) experts appended to the routed ones: expert ids
// E_routed .. E_routed + n - 1, each with T rows after the T*k routed rows.
struct SharedExperts {
  int n = 0;
  const void* w1 = nullptr;  // [n][f][d]
  const void* w3 = nullptr;  // [n][f][d]
  const void* w2 = nullptr;  // [n][d][f]
  int E_routed = 0;
};

int choose_gemm_regime(int64_t T, int k, int E);
int regime_block_rows(int regime);
// queues: the 256-row forms take their tiles from the plan's tile queues
// (n_mblocks must then head a plan piece of kPlanWords words, zeroed by the
// kernel that wrote the plan); otherwise every workgroup takes a fixed share.
hipError_t launch_fc1(int dtype, int regime, const void* x, const int32_t* perm, int k, int64_t T,
                      const void* w1, const void* w3, void* h, const int4* mblocks,
                      const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f,
                      const SharedExperts& sh, float* partial, size_t partial_bytes, bool packed, bool queues,
                      hipStream_t s);
hipError_t launch_fc2(int dtype, int regime, const void* h, const void* w2, void* y, const int4* mblocks,
                      const int32_t* n_mblocks, int64_t max_mb, int64_t est_mb, int64_t d, int64_t f,
                      const SharedExperts& sh, float* partial, size_t partial_bytes, bool packed, bool queues,
                      hipStream_t s);
// Forward weights in stage order (packed = true above): each of w1, w3, w2
// re-laid within its own E x N x K footprint (bf16, N, K multiples of 64).
hipError_t launch_pack_weights(const void* w1, const void* w3, const void* w2, void* w1p, void* w3p, void* w2p,
                               int64_t E, int64_t d, int64_t f, hipStream_t s);
// The same stage order from input-major weights w1t, w3t [E][d][f], w2t [E][f][d].
hipError_t launch_pack_weights_t(const void* w1t, const void* w3t, const void* w2t, void* w1p, void* w3p, void* w2p,
                                 int64_t E, int64_t d, int64_t f, hipStream_t s);
// bytes of the split-K partial buffer a forward FFN of this shape can use (0:
// its launches never split)
size_t splitk_partial_bytes(int dtype, int regime, int64_t max_mb, int64_t d, int64_t f);

// FC1, FC2 and the combine in one persistent launch with device-side
// readiness counters (bf16), with the tile form, weight layout (packed: stage
// order) and K split that launch_fc1 / launch_fc2 take for the same regime
// and partial buffer. sync: fused_sync_words(max_mb) int32, zero on entry;
// word kFusedErrorWord gets bit 0 set when a readiness wait gave up after
// spin_limit polls (< 0: at once).
size_t fused_sync_words(int64_t max_mb);
constexpr int kFusedErrorWord = 9;
constexpr int kFusedSpinLimit = 1 << 18;  // polls about a microsecond apart: a quarter of a second
// every workgroup of the fused launch for this shape can be resident at once
bool ffn_fused_coresident(int regime, bool packed, int64_t max_mb, int64_t est_mb, int64_t d, int64_t f,
                          size_t partial_bytes);
// Route and dispatch as the fused launch's first phases (bf16, no shared
// experts, E <= 64, T*k <= kFusedMaxAssign): the launch then writes the
// routing outputs and the plan itself, and the m-block count ends up at
// n_mblocks as after a dispatch launch.
struct FusedFront {
  bool on = false;
  const void* wg = nullptr;
  const float* bias = nullptr;
  float* logits = nullptr;
  int32_t* topk_idx = nullptr;
  float* topk_w = nullptr;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* perm = nullptr;
  int32_t* inv_perm = nullptr;
  int E = 0;
};
bool fused_front_ok(int64_t T, int E, int k);
hipError_t launch_ffn_fused(int regime, bool packed, const void* x, const int32_t* perm, int k, int64_t T,
                            const void* w1, const void* w3, const void* w2, void* h, void* y, int4* mblocks,
                            int32_t* n_mblocks, int64_t max_mb, int64_t est_mb, int64_t d, int64_t f,
                            const int32_t* inv_perm, const float* topk_w, void* out, int32_t* sync,
                            const SharedExperts& sh, float* partial, size_t partial_bytes, int spin_limit,
                            const FusedFront& front, hipStream_t s);

// Weighted combine.
// With n_shared > 0, out[t] also adds y[T*k + s*T + t] for s ascending.
hipError_t launch_combine(int dtype, const void* y, const int32_t* inv_perm, const float* w,
                          void* out, int64_t T, int64_t d, int k, hipStream_t s, int n_shared = 0);

// ---------------- backward (bf16; d and f multiples of 256) ----------------
// FC1 with g | u kept: gu [rows][2f] bf16 side by side (the backward's
// recompute), and, with h non-null, h [rows][f] bf16 = SiLU(g) u from the
// fp32 sums, as the plain FC1 forms it (the training forward).
hipError_t launch_fc1_gu(const void* x, const int32_t* perm, int k, int64_t T, const void* w1, const void* w3,
                         void* gu, const int4* mblocks, const int32_t* n_mblocks, int64_t max_mb, int64_t d,
                         int64_t f, hipStream_t s, void* h = nullptr);
// q[p] = dout[token(p)] W2_e (w2 as stored, [E][d][f], read through transposing LDS loads), fp32 [rows][f].
hipError_t launch_bwd_q(const void* dout, const int32_t* perm, int k, int64_t T, const void* w2, float* q,
                        const int4* mblocks, const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f,
                        hipStream_t s);
// dxs[p] = dg[p] W1_e + du[p] W3_e (w1, w3 as stored, [E][f][d]; two launches), fp32 [rows][d].
hipError_t launch_bwd_dx(const void* dgu, const void* w1, const void* w3, float* dxs, const int4* mblocks,
                         const int32_t* n_mblocks, int64_t max_mb, int64_t d, int64_t f, hipStream_t s);
// Weight gradients C_e = A_e B_e^T over expert e's padded K window [kofs[e], kofs[e+1]);
// A [M][pitch], B [N][pitch] bf16; output rows >= split go to c2. M, N multiples of 256.
// c and c2 fp32, or bf16 (the fp32 sums rounded to nearest even) with out_bf16.
hipError_t launch_wgrad(const void* at, const void* bt, void* c, void* c2, const int32_t* kofs, int64_t pitch,
                        int E, int64_t M, int64_t N, int64_t split, hipStream_t s, bool out_bf16 = false);
hipError_t launch_colmap(const int32_t* counts, const int32_t* offsets, int E, int64_t rows, int64_t cols,
                         int32_t* kofs, int32_t* colmap, hipStream_t s);
// mode 0: rows of src (x or dout) by token, 2: w * SiLU(g) u from gu, 3: dgu rows.
hipError_t launch_gather_transpose(int mode, const void* src, const int32_t* colmap, const int32_t* perm,
                                   const float* topk_w, int k, int64_t n_assign, int64_t F, int64_t src_pitch,
                                   void* out, int64_t cols, hipStream_t s);
hipError_t launch_swiglu_bwd(const float* q, const void* gu, const int32_t* perm, const float* topk_w, int64_t P,
                             int64_t f, void* dgu, float* dwp, hipStream_t s);
hipError_t launch_route_bwd(const int32_t* idx, const float* topk_w, const int32_t* inv_perm, const float* dwp,
                            int64_t T, int k, int E, float* dl, float* dtopk_w, float* dlogits, hipStream_t s);
hipError_t launch_dx_combine(const float* dxs, const int32_t* inv_perm, const int32_t* idx, const float* dl,
                             const void* wg, int64_t T, int k, int E, int64_t d, void* dx, hipStream_t s);
int gate_parts();
hipError_t launch_gate_grad(const void* x, const int32_t* perm, const int32_t* offsets, const float* dl, int64_t T,
                            int k, int64_t d, int E, float* part, float* bpart, float* dwg, float* dbias,
                            hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

int device_cu_count();

}  // namespace moe
