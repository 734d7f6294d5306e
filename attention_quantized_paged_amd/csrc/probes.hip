// Measurement references for the rooflines, built as a small library of their own
// (libaqp_probe.so, loaded by bench.py only); not part of the aqp ABI.
//
//  * MFMA loop: every wave issues independent bf16 MFMAs back to back (NACC accumulators in
//    round robin, so no instruction waits on the one before it), in the 16x16x32 or the
//    32x32x16 shape. Each wave also reads the shader-clock counter (s_memtime) and the
//    constant 100 MHz counter (s_memrealtime) at its start and end, so the host can divide
//    the cycles by the elapsed time: the clock the part actually held under matrix load.
//  * Gather: reads a list of pages (byte offsets into one buffer, each `page_bytes` long, a
//    multiple of 1 KB) with plain 16-byte vector loads; wave w takes the contiguous run
//    [w * per, (w + 1) * per) of the list, with `inflight` pages' loads issued before the
//    first is consumed. With the decode batch's K and V pages in the decode's order, this is
//    the achievable rate of that access pattern.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x4 __attribute__((ext_vector_type(4)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

// out: per wave (blockIdx, wave): [sum, t0_clk, t1_clk, t0_ref, t1_ref] as 5 x 8 bytes
template <int SHAPE, int NACC>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, uint64_t* out) {
  const int lane = threadIdx.x & 63;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  probe_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(2e-3f * (float)(lane - i));
  }
  float s = 0.0f;
  if constexpr (SHAPE == 16) {
    probe_f32x4 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = probe_f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    probe_f32x16 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  // lane 0 records the wave's clocks and its sum (which depends on every MFMA: each one takes
  // all lanes' operands), so no product is dead
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (lane == 0) {
    uint64_t* o = out + 5 * w;
    o[0] = (uint64_t)__builtin_bit_cast(uint32_t, s);
    o[1] = c0;
    o[2] = c1;
    o[3] = r0;
    o[4] = r1;
  }
}

// blocks work-groups of 4 waves, each wave iters x nacc MFMAs; shape 16: 16x16x32 (16384 flops
// each), 32: 32x32x16 (32768 flops each); nacc 8 or 16. out: device uint64 [blocks * 4 * 5].
// Returns 0, or -1 on bad arguments or a launch error.
extern "C" int aqp_probe_mfma_loop(int32_t shape, int32_t nacc, int32_t blocks, int32_t iters, uint64_t* out,
                                   void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  const hipStream_t st = (hipStream_t)stream;
  if (shape == 16 && nacc == 8) hipLaunchKernelGGL((mfma_loop_kernel<16, 8>), dim3(blocks), dim3(256), 0, st, iters, out);
  else if (shape == 16 && nacc == 16) hipLaunchKernelGGL((mfma_loop_kernel<16, 16>), dim3(blocks), dim3(256), 0, st, iters, out);
  else if (shape == 32 && nacc == 4) hipLaunchKernelGGL((mfma_loop_kernel<32, 4>), dim3(blocks), dim3(256), 0, st, iters, out);
  else if (shape == 32 && nacc == 8) hipLaunchKernelGGL((mfma_loop_kernel<32, 8>), dim3(blocks), dim3(256), 0, st, iters, out);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Gather: PB = page bytes / 1024 loads of 16 bytes per lane per page, IF pages in flight.
template <int PB, int IF>
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* base, const int64_t* pages, int64_t npages,
                                                     int64_t per, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t p0 = w * per;
  const int64_t p1 = p0 + per < npages ? p0 + per : npages;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int64_t p = p0; p < p1; p += IF) {
    uint4 v[IF][PB];
#pragma unroll
    for (int i = 0; i < IF; ++i) {
      const int64_t pi = p + i < p1 ? p + i : p1 - 1;
      const uint8_t* src = base + pages[pi] + 16 * lane;
#pragma unroll
      for (int j = 0; j < PB; ++j) v[i][j] = *(const uint4*)(src + 1024 * j);
    }
#pragma unroll
    for (int i = 0; i < IF; ++i)
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        acc.x ^= v[i][j].x; acc.y ^= v[i][j].y; acc.z ^= v[i][j].z; acc.w ^= v[i][j].w;
      }
  }
  out[w * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// pages: device int64 [npages] byte offsets into base (each page in bounds); page_bytes 1024,
// 2048 or 4096; inflight 2, 4 or 8; waves = blocks * 4 (each takes ceil(npages / waves) pages);
// out: device uint32 [blocks * 256]. Returns 0 or -1.
extern "C" int aqp_probe_gather(const void* base, const int64_t* pages, int64_t npages, int32_t page_bytes,
                                int32_t inflight, int32_t blocks, uint32_t* out, void* stream) {
  if (!base || !pages || npages <= 0 || blocks <= 0 || !out) return -1;
  const int64_t waves = (int64_t)blocks * 4;
  const int64_t per = (npages + waves - 1) / waves;
  const hipStream_t st = (hipStream_t)stream;
  const uint8_t* b = (const uint8_t*)base;
#define AQP_GATHER(PB, IF)                                                                                  \
  if (page_bytes == 1024 * PB && inflight == IF) {                                                          \
    hipLaunchKernelGGL((gather_kernel<PB, IF>), dim3(blocks), dim3(256), 0, st, b, pages, npages, per, out); \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                                        \
  }
  AQP_GATHER(1, 2) AQP_GATHER(1, 4) AQP_GATHER(1, 8)
  AQP_GATHER(2, 2) AQP_GATHER(2, 4) AQP_GATHER(2, 8)
  AQP_GATHER(4, 2) AQP_GATHER(4, 4)
#undef AQP_GATHER
  return -1;
}

extern "C" int aqp_probe_cu_count(void) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return n;
}
