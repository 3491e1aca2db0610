/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of one Mixture-of-Experts layer.
 *
 * One layer call computes, for T tokens x[t] (hidden size d), E routed experts
 * (SwiGLU, FFN size f) and top-k routing:
 *
 *   l[t,e]   = x[t] . Wg[e] + bias[e]                      gate GEMM + bias
 *   S_t      = the k largest l[t,.]  (ties: lower e)         top-k
 *   w[t,j]   = softmax over the k selected logits            renormalised weights
 *   out[t]   = sum_j w[t,j] * W2_e ( SiLU(W1_e x[t]) * (W3_e x[t]) ),  e = S_t[j]
 *
 * Sources: the gating network and its routing steps (top-k, per-expert counts,
 * weight normalisation, scatter into per-expert buffers) follow MegaScale-Infer,
 * "3.2 Big-Picture Architecture" and "Supporting Implementation Details / Fused
 * Kernels"; the per-expert assignment order (token, then top-k position) follows
 * MegaFlux appendix A.2; tile-aligned token blocks follow MegaFlux section 3.1;
 * the SwiGLU expert (gate, up and down matrices) follows Piper section III-A.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All pointers are DEVICE pointers unless stated otherwise; `dims` is a HOST
 *   pointer. The caller owns every buffer; the library never allocates device
 *   memory and keeps no pointer after the call returns.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream). Buffers must stay valid until the stream has passed the call.
 * - Arguments are validated on the host before anything is enqueued. On an
 *   invalid argument nothing is launched and a nonzero moe_status_t comes back.
 *   Faults during execution surface at the caller's next synchronisation.
 * - Layouts are row-major; "[a][b]" lists dimensions outermost first. Weights
 *   use the linear-layer layout [out][in] per expert.
 * - dtype MOE_DTYPE_BF16: x, Wg, W1, W3, W2, the intermediate h, y_sorted and
 *   out are bf16 (fp32 accumulation, round-to-nearest-even stores).
 *   dtype MOE_DTYPE_F32: all of them are fp32. bias, logits and topk_w are fp32
 *   in both cases; indices and counts are int32.
 * - Assignment a = t*k + j (token t, slot j). Sorted position p orders the
 *   assignments by expert, then by a.
 * - Shape limits: T >= 0 (T = 0 is a no-op), d >= 1, f >= 1, 1 <= k <= E <= 1024,
 *   T*k < 2^31, T*E < 2^31. The GPU path needs d % 64 == 0 and f % 64 == 0,
 *   and x (T*d), h (T*k*f) and one expert matrix (d*f) each under 4 GiB
 *   (MOE_ERR_UNSUPPORTED otherwise; moe_route alone accepts d % 8 == 0).
 *   Device pointers to bf16/fp32 tensors must be 16-byte aligned.
 * - Non-finite inputs give unspecified results.
 * - Thread safety: calls are independent except for the stage-timing state,
 *   which is process-wide.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1
} moe_dtype_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* null pointer, bad shape, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,  /* valid shape the GPU path does not run (see limits) */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes below what the call needs */
  MOE_ERR_HIP = 4,          /* a HIP launch or runtime call failed */
  MOE_ERR_SCRATCH = 5       /* moe_layer_forward_noalloc: the shape needs more than its static scratch */
} moe_status_t;

typedef struct {
  int64_t T;     /* tokens */
  int64_t d;     /* hidden size */
  int64_t f;     /* expert FFN size */
  int32_t E;     /* routed experts */
  int32_t k;     /* experts per token */
  int32_t dtype; /* moe_dtype_t */
} moe_dims_t;

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

/* Static text for a status code; never NULL. */
const char* moe_status_string(int status);

/* Workspace bytes that make every call below succeed for `dims` (the maximum
 * over the calls; moe_layer_forward with every optional output NULL needs the
 * most). 0 if dims is invalid. The workspace must be 256-byte aligned. */
size_t moe_workspace_bytes(const moe_dims_t* dims);

/* Rows per m-block (the tile-aligned token blocks of at most beta rows that
 * the grouped FFN's tiles cover; MegaFlux section 3.1) that moe_grouped_ffn and
 * moe_layer_forward use for `dims`: 128 when the batch has few rows per active
 * expert (96 or fewer on average, decode batches) or the data is fp32, else 256.
 * The MOE_GEMM_REGIME environment switch overrides the choice. 0 if dims is
 * invalid. Host-only query: no device work. */
int moe_ffn_block_rows(const moe_dims_t* dims);

/* Whether the gate GEMM (MegaScale-Infer, Fused Kernels, step 1) of `dims`
 * runs on the fp32 matrix cores (1) or the vector ALUs (0); -1 if dims is
 * invalid. Both give the same logits, bit for bit. The matrix cores take bf16
 * batches with d a multiple of 64, E >= 32 and at least 256 tiles of 32 tokens
 * x 32 experts; the MOE_GATE_CFG environment switch overrides ("mfma" forces
 * them where they can run, a VALU tile name forces the VALU). Host-only query:
 * no device work. */
int moe_gate_on_matrix_cores(const moe_dims_t* dims);

/* Gate GEMM + bias, top-k selection and renormalised weights
 * (MegaScale-Infer, Fused Kernels, steps 1 and 3).
 *   x      [T][d]   tokens
 *   wg     [E][d]   gate weight
 *   bias   [E] fp32 per-expert gate-logit bias, or NULL for none
 *   logits [T][E] fp32 output, or NULL (then kept in ws)
 *   topk_idx [T][k] int32 output: slot j = expert with the j-th largest logit
 *   topk_w   [T][k] fp32 output: exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * Logits are bit-reproducible: each is the fp32 sum of the products
 * x[t,i]*Wg[e,i] in a fixed order -- 64 lane classes i mod 64, each summed in
 * increasing i from +0.0, then a butterfly over offsets 32,16,8,4,2,1, then
 * one add of bias[e] -- with fp32 products rounded before each add. */
int moe_route(const moe_dims_t* dims, const void* x, const void* wg, const float* bias,
              float* logits, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, void* stream);

/* Dispatch: per-expert histogram, exclusive scan and stable permutation
 * (MegaScale-Infer, Fused Kernels, steps 2 and 4; MegaFlux appendix A.2).
 *   topk_idx [T][k] int32 input, every entry in [0, E)
 *   counts   [E]    rows per expert
 *   offsets  [E+1]  exclusive prefix sum; offsets[E] = T*k
 *   perm     [T*k]  perm[p] = a
 *   inv_perm [T*k]  inv_perm[a] = p
 * Out-of-range expert ids in topk_idx give unspecified (in-bounds) output. */
int moe_permute(const moe_dims_t* dims, const int32_t* topk_idx, int32_t* counts,
                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU expert FFN over the sorted rows (Piper, section III-A;
 * MegaFlux, sections 2.1 and 3.1): for each sorted row p of expert e,
 * with t = perm[p] / k,
 *   h[p]        = SiLU(W1_e x[t]) * (W3_e x[t])      (h rounded to dtype, kept in ws)
 *   y_sorted[p] = W2_e h[p]
 *   x [T][d]; w1, w3 [E][f][d]; w2 [E][d][f]; y_sorted [T*k][d] output.
 * perm, counts, offsets as produced by moe_permute. */
int moe_grouped_ffn(const moe_dims_t* dims, const void* x, const int32_t* perm,
                    const int32_t* counts, const int32_t* offsets,
                    const void* w1, const void* w3, const void* w2, void* y_sorted,
                    void* ws, size_t ws_bytes, void* stream);

/* Weighted combine (MegaFlux section 2.1, the separate final top-k sum):
 *   out[t] = sum_{j ascending} topk_w[t][j] * y_sorted[inv_perm[t*k+j]]
 * accumulated in fp32, stored in dtype. out [T][d]. */
int moe_combine(const moe_dims_t* dims, const void* y_sorted, const int32_t* inv_perm,
                const float* topk_w, void* out, void* stream);

/* The whole layer: route -> permute -> grouped FFN -> combine, all on `stream`,
 * with no host synchronisation. The sequence of steps follows the pages: the
 * gating network picks each token's experts and its routing steps (top-k,
 * per-expert counts, weight normalisation, scatter into per-expert order) run
 * before the experts (MegaScale-Infer, "3.2 Big-Picture Architecture" item 2
 * and "Supporting Implementation Details / Fused Kernels"); each expert's rows
 * go through FC1 then FC2 in tile-aligned token blocks, and the final top-k
 * sum is a step of its own (MegaFlux, sections 2.1 and 3.1); the expert is the
 * SwiGLU FFN of Piper, section III-A.
 *   x [T][d]; wg [E][d]; bias [E] fp32 or NULL; w1, w3 [E][f][d]; w2 [E][d][f];
 *   out [T][d] output (dtype of x).
 * logits, topk_idx, topk_w, counts, offsets, perm and inv_perm are optional
 * outputs with the layouts of moe_route and moe_permute (NULL = kept in ws).
 * ws: device workspace of at least moe_workspace_bytes(dims) bytes, 256-byte
 * aligned, owned by the caller; its contents need not be initialised and are
 * scratch after the call (moe_layer_plan_layout says where the tile plan is).
 * Errors: MOE_ERR_INVALID (null or misaligned pointer, bad dims),
 * MOE_ERR_UNSUPPORTED (shape limits above), MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
int moe_layer_forward(const moe_dims_t* dims, const void* x, const void* wg, const float* bias,
                      const void* w1, const void* w3, const void* w2, void* out,
                      float* logits, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                      void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same launches, arguments (minus ws and ws_bytes), outputs and bits as
 * moe_layer_forward, with the workspace taken from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends. The call allocates nothing: no hipMalloc or
 * allocating library routine. Shapes whose workspace
 * (moe_workspace_bytes) exceeds that size are refused with MOE_ERR_SCRATCH
 * before anything is enqueued; 128 MiB covers a Mixtral-8x22B-shaped layer
 * of up to about 700 tokens. Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (on different streams, or
 * from different threads) race and give undefined results; serialise them.
 * The first call on a device looks up the array's address there. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int moe_layer_forward_noalloc(const moe_dims_t* dims, const void* x, const void* wg, const float* bias,
                              const void* w1, const void* w3, const void* w2, void* out, float* logits,
                              int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, void* stream);

/* Shared (always-active) experts: a layer whose tokens each also pass through
 * n_shared SwiGLU experts of the same sizes outside the routing (Piper, Table III
 * notation; DeepSeek-V3: 256 routed + 1 shared, Piper Table I, note b):
 *   out[t] = sum_j w[t,j] * FFN_{S_t[j]}(x[t]) + sum_{s ascending} FFN^shared_s(x[t])
 * with weight 1 for the shared experts (not part of the renormalised softmax).
 *   sw1, sw3 [n_shared][f][d], sw2 [n_shared][d][f]: shared expert weights.
 * The routed and shared rows run in one grouped FFN (shared rows after the
 * T*k routed ones). Other arguments and outputs as moe_layer_forward (the
 * routing outputs cover the routed experts only). 1 <= n_shared and
 * E + n_shared <= 1024, else MOE_ERR_INVALID. */
size_t moe_workspace_bytes_shared(const moe_dims_t* dims, int n_shared);
int moe_layer_forward_shared(const moe_dims_t* dims, int n_shared, const void* x, const void* wg,
                             const float* bias, const void* w1, const void* w3, const void* w2,
                             const void* sw1, const void* sw3, const void* sw2, void* out,
                             float* logits, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                             void* ws, size_t ws_bytes, void* stream);

/* The same layer in one persistent launch. Workgroups take tiles from
 * device-side sequences: route tiles (one token: its logits, top-k and
 * weights), then, once the workgroup that stored the last route tile has run
 * the dispatch and written the tile plan, FC1 tiles, FC2 tiles and blocks of
 * 512 output vectors for the combine (a batch of at most 16 logits, T*E <=
 * 16, is routed and dispatched by every workgroup for itself, with no wait);
 * an FC2 tile starts once every FC1 tile of its
 * block of rows is stored, the combine once every FC2 tile is, tracked by
 * readiness counters in the workspace instead of kernel boundaries
 * (MegaScale-Infer, "Fused Kernels": the small routing steps fused; MegaFlux,
 * section 2.1: MegaMoE's tiled FC1/FC2 in one persistent kernel). Route and
 * dispatch run inside the launch when E <= 64 and T*k <= 65536 (else as
 * separate launches before it; the MOE_FUSED_FRONT=0 environment switch
 * forces that). The tiles are those of moe_layer_forward: the same rows per
 * block, FC2 tile width and the same split of K (of every tile when a
 * launch has fewer tiles than compute units, of FC2's last partial round of
 * tiles at prefill sizes; the workgroup that stores a split tile's last part
 * sums the parts in the same order), so the outputs and
 * routing arrays are bitwise equal. bf16 only (MOE_ERR_UNSUPPORTED
 * otherwise); other arguments, limits and the workspace size
 * (moe_workspace_bytes) as moe_layer_forward. */
int moe_layer_forward_fused(const moe_dims_t* dims, const void* x, const void* wg, const float* bias,
                            const void* w1, const void* w3, const void* w2, void* out, float* logits,
                            int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                            int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);
/* Readiness of the fused launch. Its waits need every workgroup of the grid
 * resident at once (persistent workgroups, MegaFlux section 2.1);
 * moe_layer_forward_fused checks the occupancy on the host and returns
 * MOE_ERR_UNSUPPORTED, enqueueing nothing, when the grid cannot all be
 * resident. Each wait is still bounded: a workgroup that polled a readiness
 * counter too long (another kernel holding CUs, for instance) gives up, sets
 * an error word in the workspace and carries on, so the launch always ends but
 * its outputs are then wrong. moe_fused_status waits for `stream` and copies
 * that word of the last moe_layer_forward_fused call on `ws` (same dims) to
 * *flags (host pointer): 0 = every wait was met, so the outputs are valid;
 * nonzero = some wait gave up, discard the outputs (bit 0: a wait for FC1 or
 * FC2 tiles; bit 1: a wait for the tile plan, after which that workgroup left
 * the launch). The word is cleared at the start of every fused call. T == 0
 * gives *flags = 0. Errors as for the workspace checks of moe_layer_forward;
 * MOE_ERR_HIP if the copy fails. */
int moe_fused_status(const moe_dims_t* dims, const void* ws, size_t ws_bytes, int32_t* flags, void* stream);

/* Where the tile plan of a layer call sits in its workspace (host-only query,
 * no device work). After moe_layer_forward, _packed, _fused or (with the same
 * n_shared) _shared on `ws`, bytes [mblocks_offset, + 16 * count) of ws hold
 * the m-blocks the grouped FFN's tiles covered -- tile-aligned token blocks of
 * at most moe_ffn_block_rows rows, at most one partial block per expert
 * (MegaFlux, section 3.1) -- and the int32 at count_offset holds count
 * (<= *max_mblocks), and the int32 after it is 1 if some expert's rows span
 * more than one m-block, else 0 (the grouped FFN's 256-row launches then take
 * their tiles from per-XCD queues). Each m-block is four int32: expert, first sorted row,
 * rows, and (first m-block of its tile group << 4) | group size (the runs of
 * up to 8 m-blocks of one expert the GEMM walks together). n_shared = 0 for
 * layers without shared experts. MOE_ERR_INVALID for bad dims, a null
 * output pointer or n_shared out of range. */
int moe_layer_plan_layout(const moe_dims_t* dims, int n_shared, size_t* mblocks_offset, size_t* count_offset,
                          int64_t* max_mblocks);

/* Expert weights re-laid in the order the grouped FFN streams them (no
 * arithmetic: a permutation of each expert matrix's bf16 values). The expert
 * FFN's FC1/FC2 tiles (MegaFlux, section 2.1) read a column block of weight
 * rows one 64-wide K step at a time, 128 bytes from each of hundreds of rows;
 * in this order every 64-row group of a matrix is K/64 contiguous 8 KiB
 * blocks, one per K step, each already in the order the loads place it in
 * LDS, which HBM streams faster. Meant for weights that are packed once and
 * read by many calls (decode); the packing is not part of a layer call.
 *   moe_pack_weights: w1p, w3p [E][f][d] and w2p [E][d][f] (device buffers the
 *     caller owns, the sizes of w1, w3, w2, 16-byte aligned, not overlapping
 *     the inputs) receive the stage-order copies of w1, w3, w2; asynchronous
 *     on `stream`. bf16 only (MOE_ERR_UNSUPPORTED otherwise); d and f
 *     multiples of 64 as for the layer.
 *   moe_layer_forward_packed: moe_layer_forward reading the packed weights
 *     in place of w1, w3, w2; same arguments, limits, workspace and outputs,
 *     and bitwise the same result (the tiles load the same values into LDS).
 * Element (e, n, k) of a packed tensor of row length K (d for w1p, w3p; f for
 * w2p) sits at 16-byte unit (((e*N/64 + n/64) * K/64 + k/64) * 64 + n%64) * 8
 * + ((k%64)/8 ^ ((n%64)/2)%8), element k%8 of the unit. */
int moe_pack_weights(const moe_dims_t* dims, const void* w1, const void* w3, const void* w2, void* w1p,
                     void* w3p, void* w2p, void* stream);
/* moe_pack_weights for weights held in the other orientation, input-major:
 * w1t, w3t [E][d][f] and w2t [E][f][d], i.e. each expert's gate and up
 * matrices as d x f and its down matrix as f x d, as Piper section III-A
 * writes them (w1t[e][i][j] = w1[e][j][i], and so on). The outputs are the
 * same stage-order tensors w1p, w3p [E][f][d], w2p [E][d][f], bitwise equal to
 * what moe_pack_weights gives for the [out][in] tensors, so the caller never
 * transposes. Same limits, ownership and errors as moe_pack_weights (plus
 * MOE_ERR_UNSUPPORTED when E * d/64 * f/64 >= 2^31); the inputs are
 * 16-byte aligned device buffers that do not overlap the outputs. */
int moe_pack_weights_transposed(const moe_dims_t* dims, const void* w1t, const void* w3t, const void* w2t,
                                void* w1p, void* w3p, void* w2p, void* stream);
int moe_layer_forward_packed(const moe_dims_t* dims, const void* x, const void* wg, const float* bias,
                             const void* w1p, const void* w3p, const void* w2p, void* out, float* logits,
                             int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);
/* moe_layer_forward_fused reading packed weights (moe_pack_weights): the one
 * persistent launch of moe_layer_forward_fused with the weight loads of
 * moe_layer_forward_packed; bitwise the same outputs as both. Arguments,
 * limits, workspace, errors and moe_fused_status as moe_layer_forward_fused. */
int moe_layer_forward_fused_packed(const moe_dims_t* dims, const void* x, const void* wg, const float* bias,
                                   const void* w1p, const void* w3p, const void* w2p, void* out, float* logits,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                   int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* ---- backward pass ----
 * Gradients of the layer for a scalar loss whose gradient with respect to
 * `out` is `dout`. The pages name the parts (MegaFlux, section 2.1: token
 * blocks stream through DGrad and WGrad, and the final top-k sum is a step of
 * its own; section 3.2 and Figure 2); the formulas are the chain rule of the
 * forward: per assignment (t, j) of expert e with weight w,
 *   dtopk_w[t][j] = dout_t . y,   dW2_e += (w dout_t) h^T,
 *   dg = (W2_e^T w dout_t) * u * SiLU'(g),  du = (W2_e^T w dout_t) * SiLU(g),
 *   dW1_e += dg x_t^T,  dW3_e += du x_t^T,  dx_t += W1_e^T dg + W3_e^T du,
 * then the softmax over the k selected logits,
 *   dlogits[t][e_j] = w_j (dtopk_w[t][j] - sum_i w_i dtopk_w[t][i]) (0 elsewhere),
 * and the gate: dbias = column sums of dlogits, dwg = dlogits^T x,
 * dx += dlogits wg. The selection itself is piecewise constant and gets no
 * gradient.
 *
 * Inputs: the forward's inputs (bf16 only: dims->dtype must be MOE_DTYPE_BF16)
 * and its routing outputs topk_idx, topk_w, counts, offsets, perm, inv_perm
 * (exactly as moe_layer_forward or moe_route + moe_permute return them), and
 * dout [T][d] bf16. Outputs (device, caller-allocated): dx [T][d] bf16;
 * dwg [E][d], dbias [E], dw1 [E][f][d], dw3 [E][f][d], dw2 [E][d][f] fp32
 * (every entry written, zero for experts that received no rows); optional
 * (NULL to skip) dlogits [T][E] and dtopk_w [T][k] fp32.
 * FC1 is recomputed (moe_layer_forward keeps only h; moe_layer_forward_train
 * and moe_layer_backward_saved below keep g and u instead); W1, W3 and W2
 * are read as stored (the DGrad products take them through transposing LDS
 * loads, no copies). Accumulation is fp32 throughout;
 * dg, du, h and w*dout enter the matrix products as bf16. Every reduction
 * has a fixed order: results are deterministic.
 * Limits: d and f multiples of 256, else MOE_ERR_UNSUPPORTED; pointers
 * 16-byte aligned (4 for the int32 / fp32 routing arrays); ws at least
 * moe_backward_workspace_bytes(dims), 256-byte aligned. T == 0 writes zero
 * weight gradients. Asynchronous on `stream`. */
size_t moe_backward_workspace_bytes(const moe_dims_t* dims);
int moe_layer_backward(const moe_dims_t* dims, const void* x, const void* wg, const void* w1, const void* w3,
                       const void* w2, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                       const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm, const void* dout,
                       void* dx, float* dwg, float* dbias, float* dw1, float* dw3, float* dw2,
                       float* dlogits, float* dtopk_w, void* ws, size_t ws_bytes, void* stream);

/* ---- training pair: FC1's g | u kept from the forward for the backward ----
 * The backward above recomputes FC1 (g = x W1_e^T, u = x W3_e^T per sorted
 * row) because the forward keeps only h. MegaFlux (section 2.1) runs the
 * backward as its own DGrad and WGrad streams and is silent on what the
 * forward saves; this pair trades [T*k][2f] bf16 of memory for that
 * recompute (4 d f FLOP per sorted row).
 *
 * moe_layer_forward_train: moe_layer_forward (same arguments, routing outputs,
 * optional NULLs and workspace, moe_workspace_bytes) plus the output
 * gu [T*k][2f] bf16 (device, caller-allocated, 16-byte aligned; required when
 * T > 0): row p holds g then u of sorted row p (the order of perm), rounded to
 * bf16. FC1 runs over 256-row tiles of the same plan as the backward's
 * recompute, so gu is bit for bit what moe_layer_backward computes internally;
 * the same launch forms h = SiLU(g) u from the fp32 sums, as moe_layer_forward
 * does, so `out` has the plain forward's arithmetic (it can differ from
 * moe_layer_forward's in the last bf16 bit where that call sums a tile's K
 * range in parts, and is held to the same 2e-2 bar against the fp64
 * definition). bf16 only; d and f multiples of 256;
 * no shared experts; errors as moe_layer_backward's limits
 * (MOE_ERR_UNSUPPORTED) and moe_layer_forward's arguments.
 *
 * moe_layer_backward_saved: moe_layer_backward with `gu` (as written by
 * moe_layer_forward_train for the same x, W1, W3 and routing arrays) read
 * instead of recomputed; every output is bit for bit moe_layer_backward's.
 * Same workspace (moe_backward_workspace_bytes), limits and errors; gu must be
 * 16-byte aligned when T > 0 (MOE_ERR_INVALID otherwise). */
int moe_layer_forward_train(const moe_dims_t* dims, const void* x, const void* wg, const float* bias,
                            const void* w1, const void* w3, const void* w2, void* out, float* logits,
                            int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                            int32_t* perm, int32_t* inv_perm, void* gu, void* ws, size_t ws_bytes, void* stream);
int moe_layer_backward_saved(const moe_dims_t* dims, const void* x, const void* wg, const void* w1,
                             const void* w3, const void* w2, const int32_t* topk_idx, const float* topk_w,
                             const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                             const int32_t* inv_perm, const void* dout, const void* gu, void* dx, float* dwg,
                             float* dbias, float* dw1, float* dw3, float* dw2, float* dlogits, float* dtopk_w,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_layer_backward with its options in one call: `gu` NULL recomputes FC1
 * (moe_layer_backward), non-NULL reads it (moe_layer_backward_saved; 16-byte
 * aligned); `wgrad_dtype` MOE_DTYPE_F32 writes dw1, dw3, dw2 as fp32 (as those
 * two calls do), MOE_DTYPE_BF16 as bf16 [same shapes], each element the
 * round-to-nearest-even bf16 of the fp32 value the fp32 form writes. The bf16
 * form halves the bytes the weight-gradient products write (3 E d f values
 * per call), which bound them when experts receive ~100 rows (the DeepSeek
 * shape). dx, dwg, dbias, dlogits, dtopk_w are as in moe_layer_backward and
 * bitwise the same. Workspace, limits and errors as moe_layer_backward;
 * MOE_ERR_INVALID for another wgrad_dtype or a misaligned gu. */
int moe_layer_backward_ex(const moe_dims_t* dims, const void* x, const void* wg, const void* w1, const void* w3,
                          const void* w2, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                          const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm, const void* dout,
                          const void* gu, int wgrad_dtype, void* dx, float* dwg, float* dbias, void* dw1,
                          void* dw3, void* dw2, float* dlogits, float* dtopk_w, void* ws, size_t ws_bytes,
                          void* stream);

/* ---- stage timing (instrumentation; process-wide, not thread-safe) ----
 * While enabled, every kernel the library launches is bracketed by HIP events
 * recorded on the stream it is launched on. Stages: */
enum {
  MOE_STAGE_GATE = 0,     /* gate logits */
  MOE_STAGE_TOPK = 1,     /* top-k + weights */
  MOE_STAGE_HIST = 2,     /* dispatch histogram */
  MOE_STAGE_SCAN = 3,     /* dispatch scan */
  MOE_STAGE_SCATTER = 4,  /* dispatch permutation */
  MOE_STAGE_PLAN = 5,     /* tile plan */
  MOE_STAGE_FC1 = 6,      /* grouped FC1 + SiLU*mul */
  MOE_STAGE_FC2 = 7,      /* grouped FC2 */
  MOE_STAGE_COMBINE = 8,  /* weighted combine */
  MOE_STAGE_DISPATCH = 9, /* single-workgroup histogram + scan + scatter (+ tile plan) */
  MOE_STAGE_BWD_WT = 10,      /* reserved (the backward reads the weights as stored) */
  MOE_STAGE_BWD_FC1 = 11,     /* backward: FC1 recompute (g | u) */
  MOE_STAGE_BWD_DH = 12,      /* backward: DGrad of FC2 (q = dout W2) */
  MOE_STAGE_BWD_SWIGLU = 13,  /* backward: dg | du and dtopk_w */
  MOE_STAGE_BWD_ROUTE = 14,   /* backward: softmax over the selected logits */
  MOE_STAGE_BWD_DX = 15,      /* backward: DGrad of FC1 */
  MOE_STAGE_BWD_DXSUM = 16,   /* backward: per-token dx sum (+ gate part) */
  MOE_STAGE_BWD_ACT_T = 17,   /* backward: activation transposes for WGrad */
  MOE_STAGE_BWD_WG2 = 18,     /* backward: WGrad of W2 */
  MOE_STAGE_BWD_WG13 = 19,    /* backward: WGrad of W1 and W3 */
  MOE_STAGE_BWD_GATE = 20,    /* backward: gate weight and bias gradients */
  MOE_STAGE_FFN_FUSED = 21,   /* FC1 + FC2 + combine in one launch (moe_layer_forward_fused) */
  MOE_NUM_STAGES = 22
};
/* Start recording; `capacity` = launches per stage to keep (host memory only);
 * `stage_mask` = bit s set records stage s (0 = every stage). Discards
 * earlier records. */
int moe_timing_enable(int capacity, unsigned stage_mask);
/* Stop recording (records are kept until the next enable). */
int moe_timing_disable(void);
/* Synchronises on the recorded events of `stage` and returns the summed
 * kernel time in ms and the number of launches recorded. */
int moe_timing_read(int stage, double* total_ms, int* launches);

/* ---- measurement probes (diagnostic; not part of the layer) ----
 * Kernels that measure what the GPU sustains, so that achieved fractions can be
 * reported against measured ceilings next to the datasheet peaks. Asynchronous
 * on `stream`; the caller times them (e.g. with events on that stream). */
/* Compute units; the probes launch one workgroup of 8 waves on each. */
int moe_probe_cus(void);
/* Streams `bytes` (a multiple of 16, 16-byte aligned device buffer `src`)
 * through LDS: each workgroup reads a contiguous slice of bytes / CUs (rounded
 * down to 16 bytes; at most 2 GiB) with 16-byte buffer loads, three 32 KiB
 * steps in flight. sink [CUs] int32 receives one loaded byte per workgroup.
 * MOE_ERR_INVALID for a null or misaligned pointer or a bad size,
 * MOE_ERR_UNSUPPORTED if a slice would be empty or too large. */
int moe_probe_hbm_read(const void* src, size_t bytes, int32_t* sink, void* stream);
/* `iters` rounds of 32 bf16 16x16x32 MFMAs (eight independent accumulator
 * chains) in each of 8 waves per CU, register operands with varied bits only:
 * FLOP = 2*16*16*32 * 32 * 8 * iters * CUs. sink [8 * CUs] fp32 receives each
 * wave's accumulator sum. MOE_ERR_INVALID for a null sink or iters < 1. */
int moe_probe_mfma(int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
