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

// Staging: every wave copies its run of 1 KB pages (byte offsets into one buffer) into LDS, with
// `inflight` pages in flight, four ways: MODE 0 the direct global -> LDS copy
// (global_load_lds_dwordx4; the wave waits until at most inflight - 1 copies are outstanding before
// the next), MODE 1 plain 16-byte loads into registers (inflight pages loaded before the first is
// used), MODE 2 the same loads each followed, once it lands, by a 16-byte LDS write, MODE 3 the
// direct copy in the batches of MODE 1 (inflight copies issued, then one wait for all of them).
// MODES 4 and 5 read each wave's run as consecutive pages (addresses computed, no offset loads) with
// a rolling window of inflight direct copies (wait until inflight - 1 are outstanding, then copy the
// next); MODE 4 also reads one LDS word of the oldest landed page per copy and waits for that read
// (s_waitcnt lgkmcnt(0)), which shows whether the copies in flight hold that counter up. The launch's
// LDS size sets how many work-groups of 4 waves a CU holds, as in the prefill kernel.
template <int MODE, int INFL>
__global__ __launch_bounds__(256) void stage_kernel(const uint8_t* base, const int64_t* pages, int64_t npages,
                                                    int64_t per, uint32_t* out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  const int64_t p0 = w * per;
  const int64_t p1 = p0 + per < npages ? p0 + per : npages;
  uint32_t acc = 0;
  uint8_t* slot0 = sm + wave * INFL * 1024 + 16 * lane;
  if constexpr (MODE == 0) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(sm + wave * INFL * 1024);
    for (int64_t p = p0; p < p1; ++p) {
      const uint8_t* src = base + pages[p] + 16 * lane;
      const uint32_t dst = lds0 + (uint32_t)((p - p0) % INFL) * 1024u;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src) : "memory");
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INFL - 1) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    acc = *(const uint32_t*)slot0;
  } else if constexpr (MODE == 4 || MODE == 5) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(sm + wave * INFL * 1024);
    const uint8_t* src = base + p0 * 1024 + 16 * lane;
    for (int64_t p = p0; p < p1; ++p) {
      const uint32_t dst = lds0 + (uint32_t)((p - p0) % INFL) * 1024u;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src) : "memory");
      src += 1024;
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INFL - 1) : "memory");
      if constexpr (MODE == 4) {
        // the oldest copy in the window has landed; read a word of it
        uint32_t v;
        const uint32_t rd = lds0 + (uint32_t)((p - p0 + 1) % INFL) * 1024u + 16u * (uint32_t)lane;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(rd) : "memory");
        acc ^= v;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    acc ^= *(const uint32_t*)slot0;
  } else if constexpr (MODE == 3) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(sm + wave * INFL * 1024);
    for (int64_t p = p0; p < p1; p += INFL) {
      int64_t off[INFL];
#pragma unroll
      for (int i = 0; i < INFL; ++i) off[i] = pages[p + i < p1 ? p + i : p1 - 1];
#pragma unroll
      for (int i = 0; i < INFL; ++i)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds0 + 1024u * i),
                     "v"(base + off[i] + 16 * lane) : "memory");
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    acc = *(const uint32_t*)slot0;
  } else {
    for (int64_t p = p0; p < p1; p += INFL) {
      uint4 v[INFL];
#pragma unroll
      for (int i = 0; i < INFL; ++i) {
        const int64_t pi = p + i < p1 ? p + i : p1 - 1;
        v[i] = *(const uint4*)(base + pages[pi] + 16 * lane);
      }
#pragma unroll
      for (int i = 0; i < INFL; ++i) {
        if constexpr (MODE == 2) *(uint4*)(slot0 + i * 1024) = v[i];
        else acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
      }
    }
    if constexpr (MODE == 2) acc = *(const uint32_t*)slot0;
  }
  out[w * 64 + lane] = acc;
}

// pages: device int64 [npages] byte offsets into base (each 1 KB page in bounds); mode 0 .. 5 (4, 5:
// npages * 1 KB <= the buffer, pages unused);
// inflight 4, 8 or 12; waves = blocks * 4; lds_bytes >= 4 * inflight * 1024 (at most 160 KB);
// out: device uint32 [blocks * 256]. Returns 0 or -1.
extern "C" int aqp_probe_stage(const void* base, const int64_t* pages, int64_t npages, int32_t mode, int32_t inflight,
                               int32_t blocks, int32_t lds_bytes, uint32_t* out, void* stream) {
  if (!base || !pages || npages <= 0 || blocks <= 0 || !out || lds_bytes < 4 * inflight * 1024 || lds_bytes > 160 * 1024)
    return -1;
  const int64_t waves = (int64_t)blocks * 4;
  const int64_t per = (npages + waves - 1) / waves;
  const hipStream_t st = (hipStream_t)stream;
  const uint8_t* b = (const uint8_t*)base;
#define AQP_STAGE(M, IF)                                                                                   \
  if (mode == M && inflight == IF) {                                                                        \
    if (hipFuncSetAttribute((const void*)stage_kernel<M, IF>, hipFuncAttributeMaxDynamicSharedMemorySize,   \
                            lds_bytes) != hipSuccess)                                                       \
      return -1;                                                                                            \
    hipLaunchKernelGGL((stage_kernel<M, IF>), dim3(blocks), dim3(256), lds_bytes, st, b, pages, npages, per, out); \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                                        \
  }
  AQP_STAGE(0, 4) AQP_STAGE(0, 8) AQP_STAGE(0, 12)
  AQP_STAGE(1, 4) AQP_STAGE(1, 8) AQP_STAGE(1, 12)
  AQP_STAGE(2, 4) AQP_STAGE(2, 8) AQP_STAGE(2, 12)
  AQP_STAGE(3, 4) AQP_STAGE(3, 8) AQP_STAGE(3, 12)
  AQP_STAGE(4, 4) AQP_STAGE(4, 8) AQP_STAGE(4, 12)
  AQP_STAGE(5, 4) AQP_STAGE(5, 8) AQP_STAGE(5, 12)
#undef AQP_STAGE
  return -1;
}

// Which accelerator die (XCD) each work-group of a launch runs on: out[b] = the XCC_ID hardware
// register of work-group b (one 64-lane work-group per entry, lane 0 writes).
__global__ __launch_bounds__(64) void xcc_kernel(int32_t* out) {
  int id;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
  if (threadIdx.x == 0) out[blockIdx.x] = id & 0xF;
}

// out: device int32 [blocks]. Returns 0 or -1.
extern "C" int aqp_probe_xcc(int32_t blocks, int32_t* out, void* stream) {
  if (blocks <= 0 || !out) return -1;
  hipLaunchKernelGGL(xcc_kernel, dim3(blocks), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Dependent chain: every MFMA of a wave accumulates into the one accumulator of the MFMA before
// it (NACC chains interleaved), the pattern of a QK^T product over the head dimension.
template <int NACC>
__global__ __launch_bounds__(256) void mfma_chain_kernel(int32_t iters, uint64_t* out) {
  const int lane = threadIdx.x & 63;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  probe_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(2e-3f * (float)(lane - i));
  }
  probe_f32x16 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = (float)(j + e);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
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

// blocks work-groups of 4 waves, each wave iters x 8 x nacc dependent 32x32x16 MFMAs (nacc 1 or 2
// chains); out as for aqp_probe_mfma_loop.
extern "C" int aqp_probe_mfma_chain(int32_t nacc, int32_t blocks, int32_t iters, uint64_t* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  const hipStream_t st = (hipStream_t)stream;
  if (nacc == 1) hipLaunchKernelGGL((mfma_chain_kernel<1>), dim3(blocks), dim3(256), 0, st, iters, out);
  else if (nacc == 2) hipLaunchKernelGGL((mfma_chain_kernel<2>), dim3(blocks), dim3(256), 0, st, iters, out);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// MFMA and vector ALU overlap: each wave issues 32x32x16 MFMAs into NACC accumulators in turn,
// each followed by NV independent fp32 multiply-adds (eight chains in turn), so the host can see
// whether a wave's ALU instructions run under its own MFMAs (cycles per MFMA stay at the MFMA's
// own) or after them (cycles grow by the ALU instructions' issue time).
template <int NV, int NACC>
__global__ __launch_bounds__(256) void mfma_valu_kernel(int32_t iters, uint64_t* out) {
  extern __shared__ uint8_t pad_lds[];
  const int lane = threadIdx.x & 63;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  probe_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(2e-3f * (float)(lane - i));
  }
  probe_f32x16 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = (float)(j + e);
  float f[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] = (float)(lane + k);
  const float m = 1.0001f + 1e-7f * (float)iters, c = 1e-6f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < NV; ++v) f[v & 7] = __builtin_fmaf(f[v & 7], m, c);
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
#pragma unroll
  for (int k = 0; k < 8; ++k) s += f[k];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
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

// blocks work-groups of 4 waves with lds_bytes of LDS each (to set the waves per SIMD), each wave
// iters x 8 x nacc MFMAs with nv multiply-adds after each; nv 0, 4, 8, 12, 16 or 24, nacc 1 or 2;
// out as for aqp_probe_mfma_loop.
extern "C" int aqp_probe_mfma_valu(int32_t nv, int32_t nacc, int32_t blocks, int32_t iters, int32_t lds_bytes,
                                   uint64_t* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out || lds_bytes < 0 || lds_bytes > 160 * 1024) return -1;
  const hipStream_t st = (hipStream_t)stream;
#define AQP_MV(NV, NA)                                                                                          \
  if (nv == NV && nacc == NA) {                                                                                 \
    if (hipFuncSetAttribute((const void*)mfma_valu_kernel<NV, NA>, hipFuncAttributeMaxDynamicSharedMemorySize,   \
                            lds_bytes) != hipSuccess)                                                           \
      return -1;                                                                                                \
    hipLaunchKernelGGL((mfma_valu_kernel<NV, NA>), dim3(blocks), dim3(256), lds_bytes, st, iters, out);          \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                                            \
  }
  AQP_MV(0, 1) AQP_MV(4, 1) AQP_MV(8, 1) AQP_MV(12, 1) AQP_MV(16, 1) AQP_MV(24, 1)
  AQP_MV(0, 2) AQP_MV(4, 2) AQP_MV(8, 2) AQP_MV(12, 2) AQP_MV(16, 2) AQP_MV(24, 2)
#undef AQP_MV
  return -1;
}

// Operand layout of v_mfma_f32_32x32x16_bf16, for a check on the host: lane l passes A values
// a[l][j] = code(l, j, 0) and B values b[l][j] = code(l, j, 1) (small integers, exact in bf16 and in
// every fp32 sum), and out[l * 16 + i] receives result register i of lane l. One wave.
__global__ __launch_bounds__(64) void mfma32_layout_kernel(const float* av, const float* bv, float* out) {
  const int lane = threadIdx.x;
  probe_bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)av[lane * 8 + j];
    b[j] = (__bf16)bv[lane * 8 + j];
  }
  probe_f32x16 c;
#pragma unroll
  for (int e = 0; e < 16; ++e) c[e] = 0.0f;
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 16; ++e) out[lane * 16 + e] = c[e];
}

// av, bv: device float [64 * 8]; out: device float [64 * 16].
extern "C" int aqp_probe_mfma32_layout(const float* av, const float* bv, float* out, void* stream) {
  if (!av || !bv || !out) return -1;
  hipLaunchKernelGGL(mfma32_layout_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, av, bv, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// LDS read rate: every wave reads a 64 KB LDS buffer over and over, kind 0 with ds_read_b128 (lane l
// at 16 l + 1024 i: 1 KB contiguous per instruction), kind 1 with ds_read_b64_tr_b8 (16-lane
// groups over 8 rows of 256 bytes). Eight reads in flight, results XOR-folded; clocks as above.
template <int KIND>
__global__ __launch_bounds__(256) void lds_read_kernel(int32_t iters, uint64_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[65536];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 65536 / 16; i += blockDim.x)
    *(uint4*)(buf + 16 * i) = make_uint4(i, i * 3u, i * 5u, i * 7u);
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t acc = 0;
  const int wv = threadIdx.x >> 6;
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == 0) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const uint4*)(buf + ((16 * lane + 1024 * (u + 8 * wv) + 4096 * (it & 1)) & 65535));
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    } else {
      typedef int probe_i32x2 __attribute__((ext_vector_type(2)));
      typedef __attribute__((address_space(3))) probe_i32x2 probe_lds_i32x2;
      probe_i32x2 v[8];
      // group g of 16 lanes: rows 8 g' .. of a 256-byte-row tile; lanes 2i, 2i+1: halves of row i
      const int g = lane >> 4, i = (lane & 15) >> 1, hf = lane & 1;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int off = ((8 * g + i) * 256 + (((u + 8 * wv + (it & 1)) ^ i) & 15) * 16 + 8 * hf) & 65535;
        v[u] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((probe_lds_i32x2*)(buf + off));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= (uint32_t)v[u].x ^ (uint32_t)v[u].y;
    }
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
  if (lane == 0) {
    uint64_t* o = out + 5 * w;
    o[0] = acc;
    o[1] = c0;
    o[2] = c1;
    o[3] = r0;
    o[4] = r1;
  }
}

// blocks work-groups of 4 waves; kind 0: ds_read_b128, 1: ds_read_b64_tr_b8; out as above.
extern "C" int aqp_probe_lds_read(int32_t kind, int32_t blocks, int32_t iters, uint64_t* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  const hipStream_t st = (hipStream_t)stream;
  if (kind == 0) hipLaunchKernelGGL((lds_read_kernel<0>), dim3(blocks), dim3(256), 0, st, iters, out);
  else if (kind == 1) hipLaunchKernelGGL((lds_read_kernel<1>), dim3(blocks), dim3(256), 0, st, iters, out);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int aqp_probe_cu_count(void) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return n;
}
