// Weighted combine: out[t] = sum_{j ascending} w[t][j] * y_sorted[inv_perm[t*k + j]],
// plus, for shared (always-active) experts, y[T*k + s*T + t] for s ascending.
//
// The final top-k sum is its own step after the expert FFN (MegaFlux,
// section 2.1); token identity, slot and weight of every assignment are kept
// for it (MegaFlux, appendix A.2). One block per token; each thread owns
// 8 consecutive columns (one 16-byte bf16 vector), accumulates in fp32 and
// stores with round-to-nearest-even.
#include "combine_vec.h"
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombThreads = 256;

template <int kDtype>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const void* __restrict__ y,
                                                               const int32_t* __restrict__ inv_perm,
                                                               const float* __restrict__ w,
                                                               void* __restrict__ out, int64_t d,
                                                               int k, int64_t n_assign, int n_shared,
                                                               int64_t T) {
  const int64_t t = blockIdx.x;
  const int64_t nvec = d / 8;
  for (int64_t c = threadIdx.x; c < nvec; c += kCombThreads)
    combine_vec<kDtype>(y, inv_perm, w, out, d, k, n_assign, n_shared, T, t, c);
}

hipError_t launch_combine(int dtype, const void* y, const int32_t* inv_perm, const float* w,
                          void* out, int64_t T, int64_t d, int k, hipStream_t s, int n_shared) {
  const int64_t n_assign = T * k;
  if (dtype == 1)
    hipLaunchKernelGGL((combine_kernel<1>), dim3(static_cast<unsigned>(T)), dim3(kCombThreads), 0, s,
                       y, inv_perm, w, out, d, k, n_assign, n_shared, T);
  else
    hipLaunchKernelGGL((combine_kernel<0>), dim3(static_cast<unsigned>(T)), dim3(kCombThreads), 0, s,
                       y, inv_perm, w, out, d, k, n_assign, n_shared, T);
  return hipGetLastError();
}

}  // namespace moe
