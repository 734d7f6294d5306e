// Achievable dense bf16 matrix rate of the part: every wave issues independent
// 16x16x32 bf16 MFMAs back to back (eight accumulators, so no instruction waits
// on the one before it). A measurement reference for the prefill kernel's
// roofline, built as its own small library; it is not part of the aqp ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  probe_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(2e-3f * (float)(lane - i));
  }
  probe_f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = probe_f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the products live
}

// blocks work-groups of 4 waves, each wave `iters` x 8 MFMAs of 16x16x32 (16384 flops each);
// out: device float [blocks * 256]. Returns 0, or -1 on bad arguments or a launch error.
extern "C" int aqp_probe_mfma_loop(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int aqp_probe_cu_count(void) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return n;
}
