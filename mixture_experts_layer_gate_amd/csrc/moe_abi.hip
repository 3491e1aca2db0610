// C ABI of the MoE-layer library: argument validation, workspace carving,
// stage timing and the launch sequence. Declarations and the contract of each
// entry point are in include/moe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <utility>
#include <vector>

#include "moe.h"
#include "kernels.h"

namespace moe {

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ---------------- stage timing ----------------
struct Timing {
  std::mutex mu;
  bool on = false;
  int cap = 0;
  unsigned mask = 0xffffffffu;
  std::vector<hipEvent_t> ev[MOE_NUM_STAGES][2];
  int n[MOE_NUM_STAGES] = {0};
} g_timing;

struct StageScope {
  int stage;
  hipStream_t s;
  int slot = -1;
  StageScope(int st, hipStream_t stream) : stage(st), s(stream) {
    if (!g_timing.on || !((g_timing.mask >> stage) & 1u)) return;
    if (g_timing.n[stage] < g_timing.cap) {
      slot = g_timing.n[stage]++;
      (void)hipEventRecord(g_timing.ev[stage][0][slot], s);
    }
  }
  ~StageScope() {
    if (slot >= 0) (void)hipEventRecord(g_timing.ev[stage][1][slot], s);
  }
};

// ---------------- validation ----------------
// a * b * c < lim, computed without overflow (a, b, c >= 0)
bool product_below(int64_t a, int64_t b, int64_t c, int64_t lim) {
  return static_cast<__int128>(a) * b * c < static_cast<__int128>(lim);
}

int check_dims(const moe_dims_t* dm) {
  if (!dm) return MOE_ERR_INVALID;
  if (dm->T < 0 || dm->d < 1 || dm->f < 1) return MOE_ERR_INVALID;
  if (dm->d >= (int64_t(1) << 31) || dm->f >= (int64_t(1) << 31)) return MOE_ERR_INVALID;
  if (dm->k < 1 || dm->E < dm->k || dm->E > 1024) return MOE_ERR_INVALID;
  if (dm->dtype != MOE_DTYPE_F32 && dm->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID;
  // T*k and T*E below 2^31 (k, E >= 1, so T first: the products then fit in 64 bits)
  if (dm->T >= (int64_t(1) << 31)) return MOE_ERR_INVALID;
  if (dm->T * dm->k >= (int64_t(1) << 31) || dm->T * dm->E >= (int64_t(1) << 31)) return MOE_ERR_INVALID;
  // every workspace piece ([T*k][max(d, f)] fp32 at most, and the backward's
  // transposed activations) stays far inside size_t
  const int64_t wide = dm->d > dm->f ? dm->d : dm->f;
  if (!product_below(dm->T * dm->k + 64 * int64_t(dm->E) + 64, 2 * wide, 8, int64_t(1) << 60)) return MOE_ERR_INVALID;
  return MOE_OK;
}
// shared experts: 1 <= n_shared, E + n_shared <= 1024, T * (k + n_shared) < 2^31 and
// the workspace pieces of those rows inside size_t (dims already checked)
int check_shared(const moe_dims_t* dm, int n_shared) {
  if (n_shared < 1 || dm->E + n_shared > 1024) return MOE_ERR_INVALID;
  const int64_t rows = dm->T * (dm->k + int64_t(n_shared)), wide = dm->d > dm->f ? dm->d : dm->f;
  if (rows >= (int64_t(1) << 31)) return MOE_ERR_INVALID;
  if (!product_below(rows + 64 * int64_t(dm->E + n_shared) + 64, 2 * wide, 8, int64_t(1) << 60))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

int elt_bytes(const moe_dims_t* dm) { return dm->dtype == MOE_DTYPE_BF16 ? 2 : 4; }
bool ok16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool ok4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
bool ok4_or_null(const void* p) { return !p || (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// ---------------- workspace layouts ----------------
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename P>
  P* take(size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off = align_up(off + bytes);
    return p;
  }
};

struct RouteWs { float* logits; };
size_t route_ws(const moe_dims_t* dm, void* ws, bool need_logits, RouteWs* out) {
  Carver c(ws);
  RouteWs r{};
  if (need_logits) r.logits = c.take<float>(sizeof(float) * dm->T * dm->E);
  if (out) *out = r;
  return c.off;
}

struct PermuteWs { int32_t* block_hist; int chunk, n_chunks; };
size_t permute_ws(const moe_dims_t* dm, void* ws, PermuteWs* out) {
  Carver c(ws);
  PermuteWs r{};
  dispatch_chunking(dm->T * dm->k, &r.chunk, &r.n_chunks);
  r.block_hist = c.take<int32_t>(sizeof(int32_t) * size_t(r.n_chunks) * dm->E);
  if (out) *out = r;
  return c.off;
}

// Sorted rows of the grouped FFN: T*k routed rows, then T rows per shared expert.
int64_t ffn_rows(const moe_dims_t* dm, int n_shared) { return dm->T * dm->k + static_cast<int64_t>(n_shared) * dm->T; }

struct FfnWs {
  int4* mblocks; int32_t* n_mblocks; void* h; int64_t max_mb; int32_t* sync;
  float* partial; size_t partial_bytes;  // split-K parts of FC1/FC2 tiles (none when no launch can split)
  size_t mblocks_off, n_mblocks_off, sync_off;  // byte offsets of the pieces from the start of this region
};
int gemm_regime(const moe_dims_t* dm);
size_t ffn_ws(const moe_dims_t* dm, void* ws, FfnWs* out, int n_shared = 0) {
  Carver c(ws);
  FfnWs r{};
  r.max_mb = max_mblocks(ffn_rows(dm, n_shared), dm->E + n_shared);
  r.mblocks_off = c.off;
  r.mblocks = c.take<int4>(sizeof(int4) * size_t(r.max_mb));
  r.n_mblocks_off = c.off;
  r.n_mblocks = c.take<int32_t>(sizeof(int32_t) * kPlanWords);  // count + tile queues
  r.h = c.take<char>(size_t(elt_bytes(dm)) * ffn_rows(dm, n_shared) * dm->f);
  r.sync_off = c.off;
  r.sync = c.take<int32_t>(sizeof(int32_t) * fused_sync_words(r.max_mb));  // fused FFN's readiness counters
  r.partial_bytes = splitk_partial_bytes(dm->dtype, gemm_regime(dm), r.max_mb, dm->d, dm->f);
  r.partial = r.partial_bytes ? c.take<float>(r.partial_bytes) : nullptr;
  if (out) *out = r;
  return c.off;
}

struct LayerWs {
  float* logits; int32_t* idx; float* w; int32_t* counts; int32_t* offsets; int32_t* perm;
  int32_t* inv; void* y; void* sub;  // sub: start of the permute / ffn scratch (shared)
  size_t sub_off;                    // byte offset of sub from the start of the workspace
};
size_t layer_ws(const moe_dims_t* dm, void* ws, LayerWs* out, int n_shared = 0) {
  Carver c(ws);
  LayerWs r{};
  const size_t n = size_t(dm->T) * dm->k;
  r.logits = c.take<float>(sizeof(float) * dm->T * dm->E);
  r.idx = c.take<int32_t>(sizeof(int32_t) * n);
  r.w = c.take<float>(sizeof(float) * n);
  r.counts = c.take<int32_t>(sizeof(int32_t) * dm->E);
  r.offsets = c.take<int32_t>(sizeof(int32_t) * (dm->E + 1));
  r.perm = c.take<int32_t>(sizeof(int32_t) * n);
  r.inv = c.take<int32_t>(sizeof(int32_t) * n);
  r.y = c.take<char>(size_t(elt_bytes(dm)) * ffn_rows(dm, n_shared) * dm->d);
  const size_t pws = permute_ws(dm, nullptr, nullptr), fws = ffn_ws(dm, nullptr, nullptr, n_shared);
  const size_t sub = pws > fws ? pws : fws;
  r.sub_off = c.off;
  r.sub = c.take<char>(sub);
  if (out) *out = r;
  return c.off;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ---------------- static scratch of the allocation-free entry point ----------------
// One copy of this array per GPU the library runs on, held until the process
// ends. Host code never passes its name to a kernel or a copy (on the host the
// name is only a stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current, on the first moe_layer_forward_noalloc call there.
static_assert(MOE_NOALLOC_SCRATCH_BYTES % kAlign == 0, "whole 256-byte pieces");
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

struct ScratchAddr {
  std::mutex mu;
  void* ptr[64] = {};
} g_scratch;

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch.ptr[dev] = p;
  }
  *out = g_scratch.ptr[dev];
  return MOE_OK;
}

// Backward scratch. P = T*k sorted rows; pp = padded columns of the transposed
// activations (every expert's rows rounded up to a multiple of 64).
struct BwdWs {
  int4* mblocks; int32_t* n_mblocks; int64_t max_mb;
  void* gu; void* dgu;           // [P][2f] bf16
  float* q;                      // [P][f]
  float* dxs;                    // [P][d]
  float* dwp; float* dl;         // [P]
  int32_t* kofs; int32_t* colmap; int64_t pp;
  void* xgt; void* dyt;          // x and dout rows by token, transposed: [d][pp] bf16
  void* ht;                      // w * h, transposed: [f][pp] bf16
  void* dgut;                    // [2f][pp] bf16
  float* gpart; float* bpart;    // gate-gradient partials [parts][E][d], [parts][E]
};
size_t bwd_ws(const moe_dims_t* dm, void* ws, BwdWs* out) {
  Carver c(ws);
  BwdWs r{};
  const int64_t P = dm->T * dm->k, d = dm->d, f = dm->f, E = dm->E;
  r.max_mb = max_mblocks(P, dm->E);
  r.pp = (P + 63) / 64 * 64 + 64 * E;
  r.mblocks = c.take<int4>(sizeof(int4) * size_t(r.max_mb));
  r.n_mblocks = c.take<int32_t>(sizeof(int32_t) * kPlanWords);  // count + tile queues
  r.gu = c.take<char>(size_t(2) * P * 2 * f);
  r.dgu = c.take<char>(size_t(2) * P * 2 * f);
  r.q = c.take<float>(sizeof(float) * P * f);
  r.dxs = c.take<float>(sizeof(float) * P * d);
  r.dwp = c.take<float>(sizeof(float) * P);
  r.dl = c.take<float>(sizeof(float) * P);
  r.kofs = c.take<int32_t>(sizeof(int32_t) * (E + 1));
  r.colmap = c.take<int32_t>(sizeof(int32_t) * r.pp);
  r.xgt = c.take<char>(size_t(2) * d * r.pp);
  r.dyt = c.take<char>(size_t(2) * d * r.pp);
  r.ht = c.take<char>(size_t(2) * f * r.pp);
  r.dgut = c.take<char>(size_t(2) * 2 * f * r.pp);
  r.gpart = c.take<float>(sizeof(float) * gate_parts() * E * d);
  r.bpart = c.take<float>(sizeof(float) * gate_parts() * E);
  if (out) *out = r;
  return c.off;
}



// ---------------- launch sequences (arguments already validated) ----------------
int do_route(const moe_dims_t* dm, const void* x, const void* wg, const float* bias, float* logits,
             int32_t* idx, float* w, hipStream_t s) {
  if (route_small_ok(dm->T, dm->E)) {
    StageScope sc(MOE_STAGE_GATE, s);  // gate and top-k in one launch
    return hip_status(launch_route_small(dm->dtype, x, wg, bias, logits, dm->T, dm->d, dm->E, dm->k, idx, w, s));
  }
  {
    StageScope sc(MOE_STAGE_GATE, s);
    if (int st = hip_status(launch_gate_logits(dm->dtype, x, wg, bias, logits, dm->T, dm->d, dm->E, s))) return st;
  }
  StageScope sc(MOE_STAGE_TOPK, s);
  return hip_status(launch_topk(logits, dm->T, dm->E, dm->k, idx, w, s));
}

// One-workgroup dispatch (histogram, scan, scatter and plan in one launch)
// up to kFusedMaxAssign assignments; MOE_DISPATCH=split or =fused overrides.
bool use_fused_dispatch(int64_t n) {
  if (n > kFusedMaxAssign) return false;
  if (const char* env = getenv("MOE_DISPATCH")) {
    if (strcmp(env, "split") == 0) return false;
    if (strcmp(env, "fused") == 0) return true;
  }
  return true;
}

int do_permute(const moe_dims_t* dm, const int32_t* idx, int32_t* counts, int32_t* offsets,
               int32_t* perm, int32_t* inv, const PermuteWs& pw, hipStream_t s) {
  const int64_t n = dm->T * dm->k;
  if (use_fused_dispatch(n)) {
    StageScope sc(MOE_STAGE_DISPATCH, s);
    return hip_status(launch_dispatch_fused(idx, n, dm->E, counts, offsets, perm, inv, 0, 0, nullptr, nullptr, s));
  }
  {
    StageScope sc(MOE_STAGE_HIST, s);
    if (int st = hip_status(launch_hist(idx, n, dm->E, pw.chunk, pw.n_chunks, pw.block_hist, s))) return st;
  }
  {
    StageScope sc(MOE_STAGE_SCAN, s);
    if (int st = hip_status(launch_scan(pw.block_hist, pw.n_chunks, dm->E, counts, offsets, s))) return st;
  }
  StageScope sc(MOE_STAGE_SCATTER, s);
  return hip_status(launch_scatter(idx, n, dm->E, pw.chunk, pw.n_chunks, pw.block_hist, perm, inv, s));
}

int gemm_regime(const moe_dims_t* dm) {
  return dm->dtype == MOE_DTYPE_BF16 ? choose_gemm_regime(dm->T, dm->k, dm->E) : 0;
}

// m-blocks expected under even routing (the list holds at most max_mb): picks
// the FC2 tile width before the counts are known on the host
int64_t expected_mblocks(const moe_dims_t* dm, int64_t br, int64_t max_mb, int n_shared) {
  const int64_t n = dm->T * dm->k, active = n < dm->E ? n : dm->E;
  int64_t est_mb = active > 0 ? active * (((n + active - 1) / active + br - 1) / br) : 1;
  est_mb += static_cast<int64_t>(n_shared) * ((dm->T + br - 1) / br);
  return est_mb < max_mb ? est_mb : max_mb;
}

// Weights in stage order are read by the large-tile kernels only
int layer_regime(const moe_dims_t* dm, bool packed) {
  const int r = gemm_regime(dm);
  return packed && r == 0 ? 1 : r;
}

int do_ffn(const moe_dims_t* dm, const void* x, const int32_t* perm, const int32_t* counts,
           const int32_t* offsets, const void* w1, const void* w3, const void* w2, void* y,
           const FfnWs& fw, hipStream_t s, bool planned = false, const SharedExperts& sh = SharedExperts{},
           bool packed = false) {
  const int regime = layer_regime(dm, packed);
  if (!planned) {
    StageScope sc(MOE_STAGE_PLAN, s);
    if (int st = hip_status(launch_plan(counts, offsets, dm->E, dm->T * dm->k, fw.max_mb, regime_block_rows(regime),
                                        fw.mblocks, fw.n_mblocks, s, sh.n, dm->T))) return st;
  }
  {
    StageScope sc(MOE_STAGE_FC1, s);
    if (int st = hip_status(launch_fc1(dm->dtype, regime, x, perm, dm->k, dm->T, w1, w3, fw.h, fw.mblocks,
                                       fw.n_mblocks, fw.max_mb, dm->d, dm->f, sh, fw.partial, fw.partial_bytes, packed,
                                       true, s)))
      return st;
  }
  StageScope sc(MOE_STAGE_FC2, s);
  return hip_status(launch_fc2(dm->dtype, regime, fw.h, w2, y, fw.mblocks, fw.n_mblocks, fw.max_mb,
                               expected_mblocks(dm, regime_block_rows(regime), fw.max_mb, sh.n), dm->d, dm->f, sh,
                               fw.partial, fw.partial_bytes, packed, true, s));
}

int do_combine(const moe_dims_t* dm, const void* y, const int32_t* inv, const float* w, void* out,
               hipStream_t s, int n_shared = 0) {
  StageScope sc(MOE_STAGE_COMBINE, s);
  return hip_status(launch_combine(dm->dtype, y, inv, w, out, dm->T, dm->d, dm->k, s, n_shared));
}

int ffn_shape_ok(const moe_dims_t* dm, int n_shared = 0) {
  if (dm->d % 64 != 0 || dm->f % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // the GEMM addresses x, h rows and one expert's weights with 32-bit byte
  // offsets, and points padding rows one row past the end of x (or of a
  // 256-row block of h), so those ends plus one row must stay below 4 GiB too
  const int64_t lim = int64_t(1) << 32, eb = elt_bytes(dm);
  if (!product_below(dm->T + 1, dm->d, eb, lim) || !product_below(dm->f, dm->d, eb, lim) ||
      !product_below(ffn_rows(dm, n_shared), dm->f, eb, lim) || !product_below(257, dm->f, eb, lim))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int bwd_shape_ok(const moe_dims_t* dm) {
  if (dm->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (dm->d % 256 != 0 || dm->f % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (int st = ffn_shape_ok(dm)) return st;
  // 32-bit byte offsets: one transposed-weight matrix per expert, the gathered
  // operands (x and dout rows, g|u and dg|du rows of a block), and the
  // transposed activations [2f][pp]
  const int64_t lim = int64_t(1) << 32, P = dm->T * dm->k, pp = (P + 63) / 64 * 64 + 64 * int64_t(dm->E);
  if (!product_below(2 * dm->f, dm->d, 2, lim) || !product_below(257 * 2, dm->f, 2, lim) ||
      !product_below(2 * dm->f, pp, 2, lim) || !product_below(dm->d, pp, 2, lim))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The layer: route, dispatch, grouped FFN over the routed (and shared) rows, combine.
// FC1, FC2 and combine as one persistent launch (the plan already in fw).
// Polls of a readiness counter before the fused launch gives up (the
// MOE_FUSED_SPIN_LIMIT environment switch overrides it; a negative value makes
// every wait give up at once, which tests use to check that the failure is reported).
int fused_spin_limit() {
  if (const char* env = getenv("MOE_FUSED_SPIN_LIMIT")) return atoi(env);
  return kFusedSpinLimit;
}

// The fused launch's regime: the separate launches' (the small-tile regime 0,
// forced through the environment only, becomes the 256-row one).
int fused_regime(const moe_dims_t* dm) { return layer_regime(dm, true); }

int do_ffn_fused(const moe_dims_t* dm, const void* x, const int32_t* perm, const int32_t* inv_perm,
                 const float* topk_w, const void* w1, const void* w3, const void* w2, void* y, void* out,
                 const FfnWs& fw, const SharedExperts& sh, hipStream_t s, bool packed,
                 const FusedFront& front = FusedFront{}) {
  const int regime = fused_regime(dm);
  const int64_t est_mb = expected_mblocks(dm, regime_block_rows(regime), fw.max_mb, sh.n);
  if (int st = hip_status(launch_fill_zero(reinterpret_cast<float*>(fw.sync),
                                           static_cast<int64_t>(fused_sync_words(fw.max_mb)), s)))
    return st;
  StageScope sc(MOE_STAGE_FFN_FUSED, s);
  return hip_status(launch_ffn_fused(regime, packed, x, perm, dm->k, dm->T, w1, w3, w2, fw.h, y, fw.mblocks,
                                     fw.n_mblocks, fw.max_mb, est_mb, dm->d, dm->f, inv_perm, topk_w, out, fw.sync, sh,
                                     fw.partial, fw.partial_bytes, fused_spin_limit(), front, s));
}

int run_layer(const moe_dims_t* dm, const SharedExperts& sh, const void* x, const void* wg, const float* bias,
              const void* w1, const void* w3, const void* w2, void* out, float* logits, int32_t* topk_idx,
              float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
              size_t ws_bytes, void* stream, bool fused = false, bool packed = false) {
  if (int st = check_dims(dm)) return st;
  if (dm->T == 0) return MOE_OK;
  if (!ok16(x) || !ok16(wg) || !ok4_or_null(bias) || !ok16(w1) || !ok16(w3) || !ok16(w2) || !ok16(out) ||
      !ok4_or_null(logits) || !ok4_or_null(topk_idx) || !ok4_or_null(topk_w) || !ok4_or_null(counts) ||
      !ok4_or_null(offsets) || !ok4_or_null(perm) || !ok4_or_null(inv_perm))
    return MOE_ERR_INVALID;
  if (int st = ffn_shape_ok(dm, sh.n)) return st;
  if (fused && dm->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return ws ? MOE_ERR_INVALID : MOE_ERR_WORKSPACE;
  if (ws_bytes < layer_ws(dm, nullptr, nullptr, sh.n)) return MOE_ERR_WORKSPACE;
  if (fused) {
    // the fused launch's readiness waits need every workgroup resident at once
    FfnWs sz{};
    ffn_ws(dm, nullptr, &sz, sh.n);
    const int regime = fused_regime(dm);
    if (!ffn_fused_coresident(regime, packed, sz.max_mb,
                              expected_mblocks(dm, regime_block_rows(regime), sz.max_mb, sh.n), dm->d, dm->f,
                              sz.partial_bytes))
      return MOE_ERR_UNSUPPORTED;
  }
  LayerWs lw{};
  layer_ws(dm, ws, &lw, sh.n);
  if (!logits) logits = lw.logits;
  if (!topk_idx) topk_idx = lw.idx;
  if (!topk_w) topk_w = lw.w;
  if (!counts) counts = lw.counts;
  if (!offsets) offsets = lw.offsets;
  if (!perm) perm = lw.perm;
  if (!inv_perm) inv_perm = lw.inv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n = dm->T * dm->k;
  FfnWs fw{};
  ffn_ws(dm, lw.sub, &fw, sh.n);
  if (fused && sh.n == 0 && fused_front_ok(dm->T, dm->E, dm->k)) {
    // route and dispatch as the fused launch's first phases
    FusedFront front;
    front.on = true;
    front.wg = wg;
    front.bias = bias;
    front.logits = logits;
    front.topk_idx = topk_idx;
    front.topk_w = topk_w;
    front.counts = counts;
    front.offsets = offsets;
    front.perm = perm;
    front.inv_perm = inv_perm;
    front.E = dm->E;
    return do_ffn_fused(dm, x, perm, inv_perm, topk_w, w1, w3, w2, lw.y, out, fw, sh, s, packed, front);
  }
  if (int st = do_route(dm, x, wg, bias, logits, topk_idx, topk_w, s)) return st;
  if (use_fused_dispatch(n)) {
    // histogram, scan, scatter (and, without shared experts, the tile plan) in one launch
    const bool plan_inline = sh.n == 0;
    {
      StageScope sc(MOE_STAGE_DISPATCH, s);
      if (int st = hip_status(launch_dispatch_fused(topk_idx, n, dm->E, counts, offsets, perm, inv_perm,
                                                    regime_block_rows(fused ? fused_regime(dm) : layer_regime(dm, packed)),
                                                    fw.max_mb,
                                                    plan_inline ? fw.mblocks : nullptr,
                                                    plan_inline ? fw.n_mblocks : nullptr, s)))
        return st;
    }
    if (fused) {
      if (!plan_inline) {
        StageScope sc(MOE_STAGE_PLAN, s);
        if (int st = hip_status(launch_plan(counts, offsets, dm->E, n, fw.max_mb, regime_block_rows(fused_regime(dm)),
                                            fw.mblocks, fw.n_mblocks, s, sh.n, dm->T)))
          return st;
      }
      return do_ffn_fused(dm, x, perm, inv_perm, topk_w, w1, w3, w2, lw.y, out, fw, sh, s, packed);
    }
    if (int st = do_ffn(dm, x, perm, counts, offsets, w1, w3, w2, lw.y, fw, s, plan_inline, sh, packed)) return st;
  } else {
    PermuteWs pw{};
    permute_ws(dm, lw.sub, &pw);
    if (int st = do_permute(dm, topk_idx, counts, offsets, perm, inv_perm, pw, s)) return st;
    if (fused) {
      {
        StageScope sc(MOE_STAGE_PLAN, s);
        if (int st = hip_status(launch_plan(counts, offsets, dm->E, n, fw.max_mb, regime_block_rows(fused_regime(dm)),
                                            fw.mblocks, fw.n_mblocks, s, sh.n, dm->T)))
          return st;
      }
      return do_ffn_fused(dm, x, perm, inv_perm, topk_w, w1, w3, w2, lw.y, out, fw, sh, s, packed);
    }
    if (int st = do_ffn(dm, x, perm, counts, offsets, w1, w3, w2, lw.y, fw, s, false, sh, packed)) return st;
  }
  return do_combine(dm, lw.y, inv_perm, topk_w, out, s, sh.n);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_version(void) { return 100; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument (null or misaligned pointer, or shape outside the limits)";
    case MOE_ERR_UNSUPPORTED: return "shape not supported by the GPU path (needs d % 64 == 0, f % 64 == 0, and x, h and one expert matrix under 4 GiB)";
    case MOE_ERR_WORKSPACE: return "workspace too small (see moe_workspace_bytes)";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_SCRATCH: return "the call needs more scratch than moe_layer_forward_noalloc's static buffer holds (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int moe_ffn_block_rows(const moe_dims_t* dm) {
  if (check_dims(dm) != MOE_OK) return 0;
  return regime_block_rows(gemm_regime(dm));
}

int moe_gate_on_matrix_cores(const moe_dims_t* dm) {
  if (check_dims(dm) != MOE_OK) return -1;
  return gate_uses_mfma(dm->dtype, dm->T, dm->d, dm->E) ? 1 : 0;
}

size_t moe_workspace_bytes(const moe_dims_t* dm) {
  if (check_dims(dm) != MOE_OK) return 0;
  size_t m = layer_ws(dm, nullptr, nullptr);
  const size_t r = route_ws(dm, nullptr, true, nullptr);
  const size_t p = permute_ws(dm, nullptr, nullptr);
  const size_t f = ffn_ws(dm, nullptr, nullptr);
  if (r > m) m = r;
  if (p > m) m = p;
  if (f > m) m = f;
  return m;
}

int moe_route(const moe_dims_t* dm, const void* x, const void* wg, const float* bias, float* logits,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (dm->T == 0) return MOE_OK;
  if (!ok16(x) || !ok16(wg) || !ok4_or_null(bias) || !ok4_or_null(logits) || !ok4(topk_idx) || !ok4(topk_w))
    return MOE_ERR_INVALID;
  if (dm->d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  RouteWs rw{};
  if (!logits) {
    if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return ws ? MOE_ERR_INVALID : MOE_ERR_WORKSPACE;
    if (ws_bytes < route_ws(dm, nullptr, true, nullptr)) return MOE_ERR_WORKSPACE;
    route_ws(dm, ws, true, &rw);
    logits = rw.logits;
  }
  return do_route(dm, x, wg, bias, logits, topk_idx, topk_w, static_cast<hipStream_t>(stream));
}

int moe_permute(const moe_dims_t* dm, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (!ok4(counts) || !ok4(offsets)) return MOE_ERR_INVALID;
  if (dm->T > 0 && (!ok4(topk_idx) || !ok4(perm) || !ok4(inv_perm))) return MOE_ERR_INVALID;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return ws ? MOE_ERR_INVALID : MOE_ERR_WORKSPACE;
  if (ws_bytes < permute_ws(dm, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
  PermuteWs pw{};
  permute_ws(dm, ws, &pw);
  return do_permute(dm, topk_idx, counts, offsets, perm, inv_perm, pw, static_cast<hipStream_t>(stream));
}

int moe_grouped_ffn(const moe_dims_t* dm, const void* x, const int32_t* perm, const int32_t* counts,
                    const int32_t* offsets, const void* w1, const void* w3, const void* w2,
                    void* y_sorted, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (dm->T == 0) return MOE_OK;
  if (!ok16(x) || !ok4(perm) || !ok4(counts) || !ok4(offsets) || !ok16(w1) || !ok16(w3) || !ok16(w2) ||
      !ok16(y_sorted))
    return MOE_ERR_INVALID;
  if (int st = ffn_shape_ok(dm)) return st;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return ws ? MOE_ERR_INVALID : MOE_ERR_WORKSPACE;
  if (ws_bytes < ffn_ws(dm, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
  FfnWs fw{};
  ffn_ws(dm, ws, &fw);
  return do_ffn(dm, x, perm, counts, offsets, w1, w3, w2, y_sorted, fw, static_cast<hipStream_t>(stream));
}

int moe_combine(const moe_dims_t* dm, const void* y_sorted, const int32_t* inv_perm, const float* topk_w,
                void* out, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (dm->T == 0) return MOE_OK;
  if (!ok16(y_sorted) || !ok4(inv_perm) || !ok4(topk_w) || !ok16(out)) return MOE_ERR_INVALID;
  if (dm->d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  return do_combine(dm, y_sorted, inv_perm, topk_w, out, static_cast<hipStream_t>(stream));
}

int moe_layer_forward(const moe_dims_t* dm, const void* x, const void* wg, const float* bias,
                      const void* w1, const void* w3, const void* w2, void* out, float* logits,
                      int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                      int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  return run_layer(dm, SharedExperts{}, x, wg, bias, w1, w3, w2, out, logits, topk_idx, topk_w, counts, offsets,
                   perm, inv_perm, ws, ws_bytes, stream);
}

int moe_layer_forward_noalloc(const moe_dims_t* dm, const void* x, const void* wg, const float* bias,
                              const void* w1, const void* w3, const void* w2, void* out, float* logits,
                              int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (dm->T == 0) return MOE_OK;
  // the workspace moe_layer_forward would need must fit the static scratch
  if (layer_ws(dm, nullptr, nullptr) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if (int st = scratch_address(&ws)) return st;
  return run_layer(dm, SharedExperts{}, x, wg, bias, w1, w3, w2, out, logits, topk_idx, topk_w, counts, offsets,
                   perm, inv_perm, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int moe_pack_weights(const moe_dims_t* dm, const void* w1, const void* w3, const void* w2, void* w1p, void* w3p,
                     void* w2p, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (dm->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (int st = ffn_shape_ok(dm)) return st;
  if (!ok16(w1) || !ok16(w3) || !ok16(w2) || !ok16(w1p) || !ok16(w3p) || !ok16(w2p)) return MOE_ERR_INVALID;
  return hip_status(
      launch_pack_weights(w1, w3, w2, w1p, w3p, w2p, dm->E, dm->d, dm->f, static_cast<hipStream_t>(stream)));
}

int moe_pack_weights_transposed(const moe_dims_t* dm, const void* w1t, const void* w3t, const void* w2t, void* w1p,
                                void* w3p, void* w2p, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (dm->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (int st = ffn_shape_ok(dm)) return st;
  if (!ok16(w1t) || !ok16(w3t) || !ok16(w2t) || !ok16(w1p) || !ok16(w3p) || !ok16(w2p)) return MOE_ERR_INVALID;
  // one workgroup per 8 KiB output block: the block count of one matrix must fit the grid
  if (int64_t(dm->E) * (dm->d / 64) * (dm->f / 64) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return hip_status(
      launch_pack_weights_t(w1t, w3t, w2t, w1p, w3p, w2p, dm->E, dm->d, dm->f, static_cast<hipStream_t>(stream)));
}

int moe_layer_forward_packed(const moe_dims_t* dm, const void* x, const void* wg, const float* bias, const void* w1p,
                             const void* w3p, const void* w2p, void* out, float* logits, int32_t* topk_idx,
                             float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                             void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (dm->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  return run_layer(dm, SharedExperts{}, x, wg, bias, w1p, w3p, w2p, out, logits, topk_idx, topk_w, counts, offsets,
                   perm, inv_perm, ws, ws_bytes, stream, false, true);
}

int moe_layer_forward_fused(const moe_dims_t* dm, const void* x, const void* wg, const float* bias,
                            const void* w1, const void* w3, const void* w2, void* out, float* logits,
                            int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                            int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  return run_layer(dm, SharedExperts{}, x, wg, bias, w1, w3, w2, out, logits, topk_idx, topk_w, counts, offsets,
                   perm, inv_perm, ws, ws_bytes, stream, true);
}

int moe_layer_forward_fused_packed(const moe_dims_t* dm, const void* x, const void* wg, const float* bias,
                                   const void* w1p, const void* w3p, const void* w2p, void* out, float* logits,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                   int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  return run_layer(dm, SharedExperts{}, x, wg, bias, w1p, w3p, w2p, out, logits, topk_idx, topk_w, counts, offsets,
                   perm, inv_perm, ws, ws_bytes, stream, true, true);
}

int moe_fused_status(const moe_dims_t* dm, const void* ws, size_t ws_bytes, int32_t* flags, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (!flags) return MOE_ERR_INVALID;
  *flags = 0;
  if (dm->T == 0) return MOE_OK;  // the layer call enqueued nothing
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return ws ? MOE_ERR_INVALID : MOE_ERR_WORKSPACE;
  if (ws_bytes < layer_ws(dm, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
  LayerWs lw{};
  layer_ws(dm, const_cast<void*>(ws), &lw);
  FfnWs fw{};
  ffn_ws(dm, lw.sub, &fw);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, fw.sync + kFusedErrorWord, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_ERR_HIP;
  *flags = v;
  return MOE_OK;
}

int moe_layer_plan_layout(const moe_dims_t* dm, int n_shared, size_t* mblocks_offset, size_t* count_offset,
                          int64_t* max_mblocks_out) {
  if (int st = check_dims(dm)) return st;
  if (!mblocks_offset || !count_offset || !max_mblocks_out) return MOE_ERR_INVALID;
  if (n_shared != 0)
    if (int st = check_shared(dm, n_shared)) return st;
  LayerWs lw{};
  layer_ws(dm, nullptr, &lw, n_shared);
  FfnWs fw{};
  ffn_ws(dm, nullptr, &fw, n_shared);
  *mblocks_offset = lw.sub_off + fw.mblocks_off;
  *count_offset = lw.sub_off + fw.n_mblocks_off;
  *max_mblocks_out = fw.max_mb;
  return MOE_OK;
}

size_t moe_workspace_bytes_shared(const moe_dims_t* dm, int n_shared) {
  if (check_dims(dm) != MOE_OK || check_shared(dm, n_shared) != MOE_OK) return 0;
  return layer_ws(dm, nullptr, nullptr, n_shared);
}

int moe_layer_forward_shared(const moe_dims_t* dm, int n_shared, const void* x, const void* wg, const float* bias,
                             const void* w1, const void* w3, const void* w2, const void* sw1, const void* sw3,
                             const void* sw2, void* out, float* logits, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                             size_t ws_bytes, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (int st = check_shared(dm, n_shared)) return st;
  if (dm->T > 0 && (!ok16(sw1) || !ok16(sw3) || !ok16(sw2))) return MOE_ERR_INVALID;
  SharedExperts sh;
  sh.n = n_shared;
  sh.w1 = sw1;
  sh.w3 = sw3;
  sh.w2 = sw2;
  sh.E_routed = dm->E;
  return run_layer(dm, sh, x, wg, bias, w1, w3, w2, out, logits, topk_idx, topk_w, counts, offsets, perm,
                   inv_perm, ws, ws_bytes, stream);
}

// The forward with FC1's g | u kept for the backward: route, dispatch, FC1 in
// its g | u form over 256-row tiles (the backward's own tile plan, so the
// stored g | u is bit for bit the backward's recompute) with h derived from
// the stored values in the same epilogue, then FC2 and the combine as in the
// plain forward.
int moe_layer_forward_train(const moe_dims_t* dm, const void* x, const void* wg, const float* bias,
                            const void* w1, const void* w3, const void* w2, void* out, float* logits,
                            int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                            int32_t* inv_perm, void* gu, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_dims(dm)) return st;
  if (int st = bwd_shape_ok(dm)) return st;
  if (dm->T == 0) return MOE_OK;
  if (!ok16(x) || !ok16(wg) || !ok4_or_null(bias) || !ok16(w1) || !ok16(w3) || !ok16(w2) || !ok16(out) ||
      !ok16(gu) || !ok4_or_null(logits) || !ok4_or_null(topk_idx) || !ok4_or_null(topk_w) ||
      !ok4_or_null(counts) || !ok4_or_null(offsets) || !ok4_or_null(perm) || !ok4_or_null(inv_perm))
    return MOE_ERR_INVALID;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return ws ? MOE_ERR_INVALID : MOE_ERR_WORKSPACE;
  if (ws_bytes < layer_ws(dm, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
  LayerWs lw{};
  layer_ws(dm, ws, &lw);
  if (!logits) logits = lw.logits;
  if (!topk_idx) topk_idx = lw.idx;
  if (!topk_w) topk_w = lw.w;
  if (!counts) counts = lw.counts;
  if (!offsets) offsets = lw.offsets;
  if (!perm) perm = lw.perm;
  if (!inv_perm) inv_perm = lw.inv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n = dm->T * dm->k;
  if (int st = do_route(dm, x, wg, bias, logits, topk_idx, topk_w, s)) return st;
  PermuteWs pw{};
  permute_ws(dm, lw.sub, &pw);
  if (int st = do_permute(dm, topk_idx, counts, offsets, perm, inv_perm, pw, s)) return st;
  FfnWs fw{};
  ffn_ws(dm, lw.sub, &fw);  // the permute scratch is dead once the permutation is written
  {
    StageScope sc(MOE_STAGE_PLAN, s);
    if (int st = hip_status(launch_plan(counts, offsets, dm->E, n, fw.max_mb, 256, fw.mblocks, fw.n_mblocks, s)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_FC1, s);
    if (int st = hip_status(launch_fc1_gu(x, perm, dm->k, dm->T, w1, w3, gu, fw.mblocks, fw.n_mblocks, fw.max_mb,
                                          dm->d, dm->f, s, fw.h)))
      return st;
  }
  const int regime = gemm_regime(dm);
  const int br = regime_block_rows(regime);
  if (br != 256) {
    StageScope sc(MOE_STAGE_PLAN, s);
    if (int st = hip_status(launch_plan(counts, offsets, dm->E, n, fw.max_mb, br, fw.mblocks, fw.n_mblocks, s)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_FC2, s);
    if (int st = hip_status(launch_fc2(dm->dtype, regime, fw.h, w2, lw.y, fw.mblocks, fw.n_mblocks, fw.max_mb,
                                       expected_mblocks(dm, br, fw.max_mb, 0), dm->d, dm->f, SharedExperts{},
                                       fw.partial, fw.partial_bytes, false, true, s)))
      return st;
  }
  return do_combine(dm, lw.y, inv_perm, topk_w, out, s);
}

size_t moe_backward_workspace_bytes(const moe_dims_t* dm) {
  if (check_dims(dm) != MOE_OK) return 0;
  return bwd_ws(dm, nullptr, nullptr);
}

// gu_saved: g | u rows kept by moe_layer_forward_train (read instead of the
// FC1 recompute), or null. wgrad_bf16: dw1, dw3, dw2 are bf16 (else fp32).
static int run_backward(const moe_dims_t* dm, const void* x, const void* wg, const void* w1, const void* w3,
                        const void* w2, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                        const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm, const void* dout,
                        void* dx, float* dwg, float* dbias, void* dw1, void* dw3, void* dw2, float* dlogits,
                        float* dtopk_w, const void* gu_saved, bool wgrad_bf16, void* ws, size_t ws_bytes,
                        void* stream) {
  if (int st = check_dims(dm)) return st;
  if (!ok16(wg) || !ok16(w1) || !ok16(w3) || !ok16(w2) || !ok16(dwg) || !ok4(dbias) || !ok16(dw1) || !ok16(dw3) ||
      !ok16(dw2) || !ok4(counts) || !ok4(offsets) || !ok4_or_null(dlogits) || !ok4_or_null(dtopk_w))
    return MOE_ERR_INVALID;
  if (dm->T > 0 && (!ok16(x) || !ok4(topk_idx) || !ok4(topk_w) || !ok4(perm) || !ok4(inv_perm) || !ok16(dout) ||
                    !ok16(dx)))
    return MOE_ERR_INVALID;
  if (int st = bwd_shape_ok(dm)) return st;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return ws ? MOE_ERR_INVALID : MOE_ERR_WORKSPACE;
  if (ws_bytes < bwd_ws(dm, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
  BwdWs b{};
  bwd_ws(dm, ws, &b);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = dm->T, d = dm->d, f = dm->f, P = T * dm->k;
  const int E = dm->E, k = dm->k;
  if (T == 0) {
    // no rows: every weight gradient is zero
    // (a bf16 gradient of n elements is n / 2 zero floats; E f d is even)
    const int64_t nw = wgrad_bf16 ? E * f * d / 2 : E * f * d;
    for (auto pr : {std::make_pair(static_cast<float*>(dw1), nw), std::make_pair(static_cast<float*>(dw3), nw),
                    std::make_pair(static_cast<float*>(dw2), nw), std::make_pair(dwg, E * d),
                    std::make_pair(dbias, int64_t(E))})
      if (int st = hip_status(launch_fill_zero(pr.first, pr.second, s))) return st;
    return MOE_OK;
  }
  {
    StageScope sc(MOE_STAGE_PLAN, s);
    if (int st = hip_status(launch_plan(counts, offsets, E, P, b.max_mb, 256, b.mblocks, b.n_mblocks, s))) return st;
  }
  if (gu_saved) {
    b.gu = const_cast<void*>(gu_saved);  // only read from here on
  } else {
    StageScope sc(MOE_STAGE_BWD_FC1, s);
    if (int st = hip_status(launch_fc1_gu(x, perm, k, T, w1, w3, b.gu, b.mblocks, b.n_mblocks, b.max_mb, d, f, s)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_DH, s);
    if (int st = hip_status(launch_bwd_q(dout, perm, k, T, w2, b.q, b.mblocks, b.n_mblocks, b.max_mb, d, f, s)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_SWIGLU, s);
    if (int st = hip_status(launch_swiglu_bwd(b.q, b.gu, perm, topk_w, P, f, b.dgu, b.dwp, s))) return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_ROUTE, s);
    if (int st = hip_status(launch_route_bwd(topk_idx, topk_w, inv_perm, b.dwp, T, k, E, b.dl, dtopk_w, dlogits, s)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_DX, s);
    if (int st = hip_status(launch_bwd_dx(b.dgu, w1, w3, b.dxs, b.mblocks, b.n_mblocks, b.max_mb, d, f, s)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_DXSUM, s);
    if (int st = hip_status(launch_dx_combine(b.dxs, inv_perm, topk_idx, b.dl, wg, T, k, E, d, dx, s))) return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_ACT_T, s);
    if (int st = hip_status(launch_colmap(counts, offsets, E, P, b.pp, b.kofs, b.colmap, s))) return st;
    if (int st = hip_status(launch_gather_transpose(0, x, b.colmap, perm, topk_w, k, P, d, d, b.xgt, b.pp, s)))
      return st;
    if (int st = hip_status(launch_gather_transpose(0, dout, b.colmap, perm, topk_w, k, P, d, d, b.dyt, b.pp, s)))
      return st;
    if (int st = hip_status(launch_gather_transpose(2, b.gu, b.colmap, perm, topk_w, k, P, f, 2 * f, b.ht, b.pp, s)))
      return st;
    if (int st = hip_status(
            launch_gather_transpose(3, b.dgu, b.colmap, perm, topk_w, k, P, 2 * f, 2 * f, b.dgut, b.pp, s)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_WG2, s);
    // dW2_e [d][f] = dout^T (w h) over expert e's rows
    if (int st = hip_status(launch_wgrad(b.dyt, b.ht, dw2, nullptr, b.kofs, b.pp, E, d, f, d, s, wgrad_bf16)))
      return st;
  }
  {
    StageScope sc(MOE_STAGE_BWD_WG13, s);
    // [dW1_e ; dW3_e] [2f][d] = [dg | du]^T x over expert e's rows
    if (int st = hip_status(launch_wgrad(b.dgut, b.xgt, dw1, dw3, b.kofs, b.pp, E, 2 * f, d, f, s, wgrad_bf16)))
      return st;
  }
  StageScope sc(MOE_STAGE_BWD_GATE, s);
  return hip_status(launch_gate_grad(x, perm, offsets, b.dl, T, k, d, E, b.gpart, b.bpart, dwg, dbias, s));
}

int moe_layer_backward(const moe_dims_t* dm, const void* x, const void* wg, const void* w1, const void* w3,
                       const void* w2, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                       const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm, const void* dout,
                       void* dx, float* dwg, float* dbias, float* dw1, float* dw3, float* dw2, float* dlogits,
                       float* dtopk_w, void* ws, size_t ws_bytes, void* stream) {
  return run_backward(dm, x, wg, w1, w3, w2, topk_idx, topk_w, counts, offsets, perm, inv_perm, dout, dx, dwg, dbias,
                      dw1, dw3, dw2, dlogits, dtopk_w, nullptr, false, ws, ws_bytes, stream);
}

int moe_layer_backward_saved(const moe_dims_t* dm, const void* x, const void* wg, const void* w1, const void* w3,
                             const void* w2, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                             const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm,
                             const void* dout, const void* gu, void* dx, float* dwg, float* dbias, float* dw1,
                             float* dw3, float* dw2, float* dlogits, float* dtopk_w, void* ws, size_t ws_bytes,
                             void* stream) {
  if (dm && dm->T > 0 && !ok16(gu)) return MOE_ERR_INVALID;
  return run_backward(dm, x, wg, w1, w3, w2, topk_idx, topk_w, counts, offsets, perm, inv_perm, dout, dx, dwg, dbias,
                      dw1, dw3, dw2, dlogits, dtopk_w, gu, false, ws, ws_bytes, stream);
}

int moe_layer_backward_ex(const moe_dims_t* dm, const void* x, const void* wg, const void* w1, const void* w3,
                          const void* w2, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                          const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm, const void* dout,
                          const void* gu, int wgrad_dtype, void* dx, float* dwg, float* dbias, void* dw1, void* dw3,
                          void* dw2, float* dlogits, float* dtopk_w, void* ws, size_t ws_bytes, void* stream) {
  if (wgrad_dtype != MOE_DTYPE_F32 && wgrad_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID;
  if (gu && (reinterpret_cast<uintptr_t>(gu) & 15)) return MOE_ERR_INVALID;
  return run_backward(dm, x, wg, w1, w3, w2, topk_idx, topk_w, counts, offsets, perm, inv_perm, dout, dx, dwg, dbias,
                      dw1, dw3, dw2, dlogits, dtopk_w, gu, wgrad_dtype == MOE_DTYPE_BF16, ws, ws_bytes, stream);
}

int moe_timing_enable(int capacity, unsigned stage_mask) {
  if (capacity < 1 || capacity > (1 << 20)) return MOE_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (int st = 0; st < MOE_NUM_STAGES; ++st)
    for (int b = 0; b < 2; ++b) {
      auto& v = g_timing.ev[st][b];
      while (static_cast<int>(v.size()) < capacity) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_HIP;
        v.push_back(e);
      }
    }
  g_timing.cap = capacity;
  g_timing.mask = stage_mask ? stage_mask : 0xffffffffu;
  for (int st = 0; st < MOE_NUM_STAGES; ++st) g_timing.n[st] = 0;
  g_timing.on = true;
  return MOE_OK;
}

int moe_timing_disable(void) {
  g_timing.on = false;
  return MOE_OK;
}

int moe_timing_read(int stage, double* total_ms, int* launches) {
  if (stage < 0 || stage >= MOE_NUM_STAGES || !total_ms || !launches) return MOE_ERR_INVALID;
  double tot = 0;
  const int n = g_timing.n[stage];
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(g_timing.ev[stage][1][i]) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0;
    if (hipEventElapsedTime(&ms, g_timing.ev[stage][0][i], g_timing.ev[stage][1][i]) != hipSuccess)
      return MOE_ERR_HIP;
    tot += ms;
  }
  *total_ms = tot;
  *launches = n;
  return MOE_OK;
}

}  // extern "C"
