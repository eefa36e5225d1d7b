// Measurement helpers, not part of the attention path: a loop of dense bf16
// MFMAs and a read stream, which give the MFMA rate and the HBM read rate this
// GPU reaches under load, so that a kernel's figure can be set against them as
// well as against the datasheet peaks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_verify.h"

namespace mlav_cal {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // four waves
constexpr int kChains = 4;      // independent accumulators per wave

// Each wave runs `iters` rounds of kChains v_mfma_f32_16x16x32_bf16, one per
// accumulator.  Lane l holds A = (l + k) / 1024 and B = (l - k) / 1024 for its
// eight k: integers times 2^-10, so each product is an integer times 2^-20 of
// at most 4,410 and each thread's sum grows by at most 2.26e6 such units per
// round; below 2^24 units (iters <= 4) every sum is exact and the result is
// linear in iters.  Each thread writes the sum of its accumulators, which
// keeps the loop from being dropped.
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)((float)(lane + k) * 0x1p-10f);
    b[k] = (__bf16)((float)(lane - k) * 0x1p-10f);
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Read stream: each thread loads 16-byte units of buf at a grid stride (each
// wave covers 1 KB contiguous per step) and writes the sum of their 32-bit
// words, so every byte is read once and nothing but `out` is written.
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const uint4* buf, int64_t units, float* out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t s0 = 0u, s1 = 0u;
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + stride < units; u += 2 * stride) {
    const uint4 x = buf[u], y = buf[u + stride];
    s0 += (x.x ^ x.y) + (x.z ^ x.w);
    s1 += (y.x ^ y.y) + (y.z ^ y.w);
  }
  if (u < units) {
    const uint4 x = buf[u];
    s0 += (x.x ^ x.y) + (x.z ^ x.w);
  }
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = (float)(s0 + s1);
}

}  // namespace mlav_cal

extern "C" mla_verify_status_t mla_verify_calibrate_mfma(int32_t iters, int32_t blocks, float* out,
                                                         void* stream) {
  if (iters < 1 || blocks < 1 || !out || (reinterpret_cast<uintptr_t>(out) & 3u))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(mlav_cal::mfma_loop_kernel, dim3((unsigned)blocks), dim3(mlav_cal::kThreads), 0,
                     (hipStream_t)stream, (int)iters, out);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

extern "C" mla_verify_status_t mla_verify_calibrate_read(const void* buf, int64_t bytes, int32_t blocks, float* out,
                                                         void* stream) {
  if (!buf || bytes < 16 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u) || blocks < 1 || !out ||
      (reinterpret_cast<uintptr_t>(out) & 3u))
    return MLA_VERIFY_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(mlav_cal::read_stream_kernel, dim3((unsigned)blocks), dim3(mlav_cal::kThreads), 0,
                     (hipStream_t)stream, reinterpret_cast<const uint4*>(buf), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}
