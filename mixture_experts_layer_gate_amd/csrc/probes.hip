// Measurement probes: what this GPU sustains, for reporting achieved fractions
// against measured ceilings next to the datasheet peaks.
//
// * hbm_read_probe: one workgroup of 8 waves per CU streams a contiguous slice
//   of a device buffer into LDS with 16-byte non-temporal buffer loads (the
//   load form of the grouped GEMM's weight stream), 32 KiB per step, three
//   steps in flight.
// * mfma_probe: 8 waves per CU each run eight independent chains of bf16
//   16x16x32 MFMAs (the GEMM's form) on register operands; no memory traffic.
//   Each wave does 4 x 8 x 16384 = 524288 FLOP per iteration.
#include <stdint.h>

#include "common.h"
#include "kernels.h"
#include "moe.h"

namespace moe {

constexpr int kProbeThreads = 512;
[[maybe_unused]] constexpr int kProbeStep = 32768;  // bytes per workgroup step
[[maybe_unused]] constexpr int kProbeSlots = 4;     // LDS step buffers

__global__ __launch_bounds__(kProbeThreads, 1) void hbm_read_probe(const char* src, uint32_t slice, int32_t* sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) char lds[kProbeSlots * kProbeStep];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(src) + static_cast<size_t>(blockIdx.x) * slice, static_cast<short>(0),
      static_cast<int>(slice), 0x00020000);
  const uint32_t steps = (slice + kProbeStep - 1) / kProbeStep;
  for (uint32_t s = 0; s < steps; ++s) {
    char* dst = lds + (s % kProbeSlots) * kProbeStep;
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // 4 x 1 KiB per wave, 32 KiB per workgroup; past the slice: zeros, no request
      const int inst = wv * 4 + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + inst * 1024), 16,
                                               s * kProbeStep + inst * 1024 + lane * 16, 0, 0, 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | 12);  // vmcnt(12): three steps of 4 loads in flight
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (tid == 0) sink[blockIdx.x] = lds[(blockIdx.x * 64) % (kProbeSlots * kProbeStep)];
#endif
}

__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe(int iters, float* sink) {
  const int tid = threadIdx.x;
  // operands with varied mantissa bits, as real activations and weights have: the
  // MFMA pipes' power, and so the clock they sustain, depends on how many bits toggle
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>((tid * 7 + i) % 13) * 0.07f - 0.4f);
    b[i] = static_cast<__bf16>(static_cast<float>((tid * 5 + i * 3) % 11) * 0.09f - 0.5f);
  }
  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[c][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) s += acc[c][v];
  if ((tid & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (tid >> 6)] = s;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_probe_cus(void) { return device_cu_count(); }

int moe_probe_hbm_read(const void* src, size_t bytes, int32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return MOE_ERR_INVALID;
  const int cus = device_cu_count();
  const size_t slice = bytes / static_cast<size_t>(cus) / 16 * 16;
  if (slice == 0 || slice >= (size_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(hbm_read_probe, dim3(cus), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(src), static_cast<uint32_t>(slice), sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_probe_mfma(int iters, float* sink, void* stream) {
  if (!sink || iters < 1) return MOE_ERR_INVALID;
  hipLaunchKernelGGL(mfma_probe, dim3(device_cu_count()), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     iters, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
