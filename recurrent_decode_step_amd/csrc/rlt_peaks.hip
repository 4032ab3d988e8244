// Achievable peaks of the part, measured on it, to price the path's kernels
// against what the hardware delivers as well as against its published
// figures: a streaming read and a copy of a caller buffer (16-byte
// non-temporal accesses, one contiguous span per workgroup), and dense MFMA
// loops (independent accumulator chains, operands in registers) for the two
// bf16 matrix instructions the kernels use.  Each launch is timed by HIP
// events bound to its own dispatch.
#include "rlt_internal.h"
#include "rlt_device.h"

#include <math.h>

namespace rlt {
namespace {

constexpr int kPeakThreads = 256;
constexpr size_t kPeakSpan = 65536;          // bytes per workgroup of the streaming kernels
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kPeakThreads) void k_peak_read(const u32x4 *__restrict__ src,
                                                            u32x4 *__restrict__ sink) {
  constexpr int PER = (int)(kPeakSpan / 16);
  const u32x4 *p = src + (size_t)blockIdx.x * PER;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
#pragma unroll 16
  for (int i = threadIdx.x; i < PER; i += kPeakThreads) acc ^= __builtin_nontemporal_load(p + i);
  // a store that depends on every load (taken with probability 2^-128)
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x2545f491u && acc.w == 0x4f6cdd1du)
    sink[threadIdx.x] = acc;
}

__global__ __launch_bounds__(kPeakThreads) void k_peak_copy(const u32x4 *__restrict__ src,
                                                            u32x4 *__restrict__ dst) {
  constexpr int PER = (int)(kPeakSpan / 16);
  const size_t base = (size_t)blockIdx.x * PER;
#pragma unroll 16
  for (int i = threadIdx.x; i < PER; i += kPeakThreads)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + base + i), dst + base + i);
}

// SHAPE 0: v_mfma_f32_32x32x16_bf16 (32768 FLOP per instruction), four chains
// per wavefront; SHAPE 1: v_mfma_f32_16x16x32_bf16 (16384 FLOP), eight chains.
template <int SHAPE>
__global__ __launch_bounds__(kPeakThreads) void k_peak_mfma(int iters, float *__restrict__ sink) {
  const unsigned lane = threadIdx.x & 63u;
  // operands that depend on the lane (not constant-folded), small normal bf16 values
  const unsigned w = 0x3f803f80u + (lane & 7u) * 0x00010001u;
  const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w, w ^ 0x00020002u, w, w ^ 0x00040004u});
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{w ^ 0x00010001u, w, w ^ 0x00030003u, w});
  float total = 0.f;
  if constexpr (SHAPE == 0) {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) total += acc[j][e];
  } else {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) total += acc[j].x + acc[j].y + acc[j].z + acc[j].w;
  }
  sink[(size_t)blockIdx.x * kPeakThreads + threadIdx.x] = total;
}

// the fastest of `reps` launches, in milliseconds (events on the dispatch)
template <typename F>
hipError_t time_min(int reps, hipStream_t s, F &&go, double *ms_min) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  double best = INFINITY;
  for (int r = 0; r < reps && err == hipSuccess; ++r) {
    err = go(e0, e1);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess && ms < best) best = ms;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  *ms_min = best;
  return err;
}

rlt_status peak_fail(hipError_t e) {
  (void)hipGetLastError();
  return e == hipErrorInvalidValue ? RLT_ERR_INVALID_ARG : RLT_ERR_DEVICE;
}

}  // namespace
}  // namespace rlt

extern "C" {

rlt_status rlt_peak_bandwidth(const void *dev_src, void *dev_dst, size_t bytes, int32_t copy,
                              int32_t reps, double *gb_per_s, void *stream) {
  using namespace rlt;
  if (!dev_src || !dev_dst || !gb_per_s || reps < 1) return RLT_ERR_INVALID_ARG;
  if (bytes < ((size_t)64 << 20) || bytes % kPeakSpan || (uintptr_t)dev_src % 16 ||
      (uintptr_t)dev_dst % 16)
    return RLT_ERR_SHAPE;
  const dim3 grid((unsigned)(bytes / kPeakSpan));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4 *src = static_cast<const u32x4 *>(dev_src);
  u32x4 *dst = static_cast<u32x4 *>(dev_dst);
  double ms = 0.0;
  const hipError_t e = time_min(reps, s, [&](hipEvent_t e0, hipEvent_t e1) {
    void *ra[] = {&src, &dst};
    return copy ? hipExtLaunchKernel(reinterpret_cast<const void *>(k_peak_copy), grid,
                                     dim3(kPeakThreads), ra, 0, s, e0, e1, 0)
                : hipExtLaunchKernel(reinterpret_cast<const void *>(k_peak_read), grid,
                                     dim3(kPeakThreads), ra, 0, s, e0, e1, 0);
  }, &ms);
  if (e != hipSuccess) return peak_fail(e);
  *gb_per_s = (double)bytes * (copy ? 2.0 : 1.0) / (ms * 1e-3) / 1e9;
  return RLT_OK;
}

rlt_status rlt_peak_mfma(int32_t shape, int32_t iters, int32_t reps, float *dev_sink,
                         size_t sink_bytes, double *tflops, void *stream) {
  using namespace rlt;
  if (!dev_sink || !tflops || reps < 1 || iters < 1 || (shape != 0 && shape != 1))
    return RLT_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return RLT_ERR_DEVICE;
  const dim3 grid((unsigned)(2 * cus));            // two workgroups of 4 wavefronts per CU
  if (sink_bytes < (size_t)grid.x * kPeakThreads * sizeof(float)) return RLT_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double ms = 0.0;
  const hipError_t e = time_min(reps, s, [&](hipEvent_t e0, hipEvent_t e1) {
    void *ra[] = {&iters, &dev_sink};
    return shape == 0 ? hipExtLaunchKernel(reinterpret_cast<const void *>(k_peak_mfma<0>), grid,
                                           dim3(kPeakThreads), ra, 0, s, e0, e1, 0)
                      : hipExtLaunchKernel(reinterpret_cast<const void *>(k_peak_mfma<1>), grid,
                                           dim3(kPeakThreads), ra, 0, s, e0, e1, 0);
  }, &ms);
  if (e != hipSuccess) return peak_fail(e);
  const double waves = (double)grid.x * (kPeakThreads / 64);
  const double flop = waves * iters * (shape == 0 ? 4.0 * 32768.0 : 8.0 * 16384.0);
  *tflops = flop / (ms * 1e-3) / 1e12;
  return RLT_OK;
}

}  // extern "C"
