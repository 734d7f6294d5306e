// Cache write: quantise bf16 K/V rows and scatter them into the paged cache.
//
// Follows the reshape-and-cache step of the "CPU backend adds FP8 KV-cache
// quantisation" page (vllm PR 39445, Implementation items 1 and 3: scalar
// float -> fp8 quantisation, one entry point taking the kv dtype and scales)
// and the dynamic per-(token, head) scales of the "Per-token-head INT8/FP8 KV
// quantisation" page (vllm PR 38378, Implementation item 3: absmax over the
// head dimension divided by the format's largest code, stored inline).
//
// Work split: a row is (K or V, token, KV head) of head_dim values; D/8
// lanes take 8 values each (one 16-byte load, one 8-byte store), so one
// wave covers 64*8/D rows of consecutive heads of one token range and both
// the loads and the page stores are contiguous per row. Each lane loads
// several rows before it converts any, so enough bytes are in flight per CU
// to cover HBM latency; the grid is one resident wave of work-groups that
// strides over the rows. The per-token-head absmax is a butterfly over the
// row's lanes (per group: over the group's lanes).
//
// Rounding: the hardware fp32 -> fp8 conversions of gfx950 round to nearest
// even; values are first clamped to the largest finite code (v_med3) so that
// overflow saturates instead of producing NaN. int8 uses v_rndne + clamp.
#include "device_common.h"

namespace aqp {

template <int DT>
__device__ __forceinline__ uint32_t encode4(float y0, float y1, float y2, float y3) {
  if constexpr (DT == AQP_KV_FP8_E4M3) {
    y0 = __builtin_amdgcn_fmed3f(y0, -448.0f, 448.0f);
    y1 = __builtin_amdgcn_fmed3f(y1, -448.0f, 448.0f);
    y2 = __builtin_amdgcn_fmed3f(y2, -448.0f, 448.0f);
    y3 = __builtin_amdgcn_fmed3f(y3, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
    return (uint32_t)w;
  } else if constexpr (DT == AQP_KV_FP8_E5M2) {
    y0 = __builtin_amdgcn_fmed3f(y0, -57344.0f, 57344.0f);
    y1 = __builtin_amdgcn_fmed3f(y1, -57344.0f, 57344.0f);
    y2 = __builtin_amdgcn_fmed3f(y2, -57344.0f, 57344.0f);
    y3 = __builtin_amdgcn_fmed3f(y3, -57344.0f, 57344.0f);
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, w, true);
    return (uint32_t)w;
  } else {
    const int i0 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(y0), -128.0f, 127.0f);
    const int i1 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(y1), -128.0f, 127.0f);
    const int i2 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(y2), -128.0f, 127.0f);
    const int i3 = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(y3), -128.0f, 127.0f);
    return (uint32_t)(i0 & 0xFF) | ((uint32_t)(i1 & 0xFF) << 8) | ((uint32_t)(i2 & 0xFF) << 16) |
           ((uint32_t)(i3 & 0xFF) << 24);
  }
}

// Max over aligned runs of SPAN lanes (SPAN = 4, 8, 16, 32), in VALU: DPP quad permutes (lane ^ 1,
// lane ^ 2), then mirrors within 8 and 16 lanes (after the quad steps every lane of a quad holds
// its maximum, so pairing quad q with its mirror covers the run), then the 16-lane row swap.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int SPAN>
__device__ __forceinline__ float max_in_span(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));                             // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));                             // quad_perm [2,3,0,1]
  if constexpr (SPAN >= 8) v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
  if constexpr (SPAN >= 16) v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  if constexpr (SPAN >= 32) {
    auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
    v = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  }
  static_assert(SPAN >= 4 && SPAN <= 32, "span");
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

template <int D, int DT, int MODE>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  constexpr int TPR = D / 8;          // lanes per row
  constexpr int RPB = 256 / TPR;      // rows per work-group and sub-pass
  constexpr int U = kCwRowsPerLane;   // rows per lane per pass, loaded together
  constexpr float QMAX = DT == AQP_KV_INT8 ? 127.0f : (DT == AQP_KV_FP8_E4M3 ? 448.0f : 57344.0f);
  const int64_t per_kv = a.num_tokens * a.num_kv_heads;
  const int64_t rows = 2 * per_kv;
  const int sub = threadIdx.x % TPR;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB * U; r0 < rows; r0 += (int64_t)gridDim.x * RPB * U) {
    // issue the U rows' loads (16 bytes of values, 8 bytes of slot each) before using any
    uint4 in[U];
    int64_t slot[U];
    int kv[U], h[U];
    bool active[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u * RPB + threadIdx.x / TPR;
      active[u] = r < rows;
      const int64_t rr = active[u] ? r : rows - 1;  // keep every lane in the row's butterfly
      kv[u] = rr >= per_kv ? 1 : 0;
      const int64_t rem = rr - kv[u] * per_kv;
      // token and head of the row: a 32-bit division whenever the rows fit (uniform branch)
      const int64_t t = a.narrow ? (int64_t)div_invariant((uint32_t)rem, a.heads_magic, a.heads_shift) : rem / a.num_kv_heads;
      h[u] = (int)(rem - t * a.num_kv_heads);
      in[u] = *(const uint4*)((kv[u] ? a.v : a.k) + t * a.token_stride + (int64_t)h[u] * D + sub * 8);
      slot[u] = a.slots[t];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[8] = {bf16_lo(in[u].x), bf16_hi(in[u].x), bf16_lo(in[u].y), bf16_hi(in[u].y),
                    bf16_lo(in[u].z), bf16_hi(in[u].z), bf16_lo(in[u].w), bf16_hi(in[u].w)};
      float s;
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD || MODE == AQP_SCALE_PER_GROUP) {
        // absmax over the row (per token-head) or over the lane's group of AQP_SCALE_GROUP
        // channels (per group: AQP_SCALE_GROUP / 8 neighbouring lanes)
        constexpr int SPAN = MODE == AQP_SCALE_PER_GROUP ? AQP_SCALE_GROUP / 8 : TPR;
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
        amax = max_in_span<SPAN>(amax);
        s = amax / QMAX;  // correctly rounded fp32 division
      } else {
        s = kv[u] ? a.v_scale : a.k_scale;
      }
      const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
      if (!active[u] || slot[u] < 0 || slot[u] >= a.total_slots) continue;
      const int64_t blk = a.narrow ? (int64_t)div_invariant((uint32_t)slot[u], a.bs_magic, a.bs_shift) : slot[u] / a.block_size;
      const int off = (int)(slot[u] - blk * a.block_size);
      uint8_t* page = a.cache + blk * a.block_bytes + (int64_t)(kv[u] * a.num_kv_heads + h[u]) * a.page_bytes;
      if constexpr (DT == AQP_KV_AUTO) {
        // the unquantised cache stores the row as given: 16 bytes in, 16 bytes out
        *(uint4*)(page + (int64_t)off * D * 2 + sub * 16) = in[u];
        continue;
      }
      uint2 codes;
      codes.x = encode4<DT>(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
      codes.y = encode4<DT>(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
      *(uint2*)(page + (int64_t)off * D + sub * 8) = codes;
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
        if (sub == 0) *(float*)(page + (int64_t)a.block_size * D + 4 * off) = s;
      }
      if constexpr (MODE == AQP_SCALE_PER_GROUP) {
        constexpr int NG = D / AQP_SCALE_GROUP;
        constexpr int SPAN = AQP_SCALE_GROUP / 8;
        if (sub % SPAN == 0) *(float*)(page + (int64_t)a.block_size * D + 4 * ((int64_t)off * NG + sub / SPAN)) = s;
      }
    }
  }
}

template <int D, int DT, int MODE>
static int launch_cw(const CacheWriteArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = 2 * a.num_tokens * a.num_kv_heads;
  int64_t grid = (rows + RPB * kCwRowsPerLane - 1) / (RPB * kCwRowsPerLane);
  const int64_t resident = (int64_t)device_cu_count() * kCwWgsPerCu;
  if (grid > resident) grid = resident;
  hipLaunchKernelGGL((cache_write_kernel<D, DT, MODE>), dim3((unsigned)grid), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("aqp_cache_write: launch failed: %s", hipGetErrorString(e));
    return AQP_ERR_HIP;
  }
  return AQP_OK;
}

template <int DT, int MODE>
static int dispatch_d(const CacheWriteArgs& a, hipStream_t st) {
  switch (a.head_dim) {
    case 64: return launch_cw<64, DT, MODE>(a, st);
    case 128: return launch_cw<128, DT, MODE>(a, st);
    case 256: return launch_cw<256, DT, MODE>(a, st);
  }
  set_error("aqp_cache_write: unsupported head_dim %d", a.head_dim);
  return AQP_ERR_UNSUPPORTED;
}

int launch_cache_write(int dtype, int mode, const CacheWriteArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_AUTO) return dispatch_d<AQP_KV_AUTO, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E4M3) return dispatch_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E5M2) return dispatch_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_INT8) return dispatch_d<AQP_KV_INT8, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E4M3) return dispatch_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_INT8) return dispatch_d<AQP_KV_INT8, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E5M2) return dispatch_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_INT8) return dispatch_d<AQP_KV_INT8, AQP_SCALE_PER_GROUP>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_FP8_E4M3) return dispatch_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_GROUP>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_FP8_E5M2) return dispatch_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_GROUP>(a, st);
  set_error("aqp_cache_write: dtype %d with scale mode %d is not built", dtype, mode);
  return AQP_ERR_UNSUPPORTED;
}

}  // namespace aqp
