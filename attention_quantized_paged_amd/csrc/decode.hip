// Decode attention (one query token per sequence) over the quantised paged
// cache, and the merge of split-KV partial results.
//
// Method: the dequantise step fused into the two products of the KV tile loop
// with an online softmax ("CPU backend adds FP8 KV-cache quantisation" page,
// vllm PR 39445, Implementation item 2 and Review: dequantise inside the tile
// GEMMs, fold the scales; "Per-token-head INT8/FP8 KV quantisation" page,
// vllm PR 38378, Implementation item 3: dequantise KV tiles inside the unified
// attention), with the scheduler's split of long key ranges ("Fix CPU FP8
// attention scheduler scratch sizing" page, vllm PR 50194: enable_kv_split).
//
// gfx950 mapping, per work-group of 4 waves and per schedule segment
// (keys [k_lo, k_hi) of one (sequence, KV head, group of <= 16 q heads)):
//  * a wave takes 32-key iterations w, w+4, ... of the segment;
//  * K: each lane loads D/4 contiguous code bytes of one key straight from HBM
//    (16 keys x D bytes of a page per tile); the codes are widened to bf16 in
//    registers and fed to v_mfma_f32_16x16x32_bf16 as S^T = K * Q^T with the
//    group's q heads as the 16 MFMA columns;
//  * scale folding: per tensor, k_scale goes into the logit scale and v_scale
//    into the final normalisation; per token-head, each key's scale multiplies
//    its logit and each value's scale its probability;
//  * softmax: running max / sum in the exp2 domain, the max reduced across the
//    four lanes that share a head with two xor shuffles;
//  * V: the two 16-key tiles of codes are staged in the wave's own LDS buffer
//    and read back with ds_read_b64_tr_b8, which hands each lane 8 keys of one
//    head-dim column: exactly the key-contiguous operand O^T = V^T * P^T needs,
//    so the probabilities stay in the registers the QK^T product left them in;
//  * the four waves' (m, l, O) are merged in LDS; the result is either the
//    output row (bf16) or a partial slot for the split-KV merge kernel.
#include "device_common.h"

namespace aqp {

struct DecArgs {
  const uint8_t* cache;
  const uint16_t* q;
  const int32_t* block_tables;
  const DecSeg* segs;
  const int32_t* wg_start;
  float* scratch;
  uint16_t* out;
  int64_t page_bytes, block_bytes;
  int32_t block_size, num_kv_heads, num_q_heads, group, max_blocks, group_heads, num_blocks, num_parts;
  float logit_scale;  // sm_scale * k_scale (per tensor) or sm_scale (per token-head)
  float softcap, inv_softcap;
  float v_scale;      // per tensor; 1 per token-head
};

template <int D, int MODE>
struct IterRegs {
  static constexpr int KV4 = D / 64;  // uint4 per lane per 16-key tile (D/4 bytes)
  uint4 ka[KV4], kb[KV4];             // K codes: tile A / tile B, one key row slice per lane
  uint4 va[KV4], vb[KV4];             // V codes: tile A / tile B, coalesced slices
  float4 ksa, ksb, vsa, vsb;          // per token-head scales of the lane's 4 keys in each tile
  bool oka, okb;                      // tile lies in a block the table maps to a valid block id
};

template <int D, int DT, int MODE>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs a) {
  constexpr int KV4 = D / 64;
  constexpr int NT = D / 16;   // 16-wide head-dim tiles of the output
  constexpr int QS = D / 32;   // 32-deep MFMA steps of QK^T
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  uint8_t* vbuf = smem + wave * (kDecIterKeys * D);
  const int s_begin = a.wg_start[blockIdx.x], s_end = a.wg_start[blockIdx.x + 1];

  for (int si = s_begin; si < s_end; ++si) {
    const DecSeg sg = a.segs[si];
    const int head = sg.head0 + r16;
    const bool head_ok = r16 < sg.nheads;
    const int hq = sg.kvh * a.group + head;
    // Q^T operand: lane (column head r16, group kg) holds q[head][kg*D/4 + 8*st + 0..7] for step st.
    bf16x8 qb[QS];
    {
      const uint16_t* qp = a.q + ((int64_t)sg.q_tok * a.num_q_heads + (head_ok ? hq : sg.kvh * a.group)) * D + kg * (D / 4);
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        uint4 u = *(const uint4*)(qp + st * 8);
        if (!head_ok) u = make_uint4(0, 0, 0, 0);
        qb[st] = __builtin_bit_cast(bf16x8, u);
      }
    }
    const int32_t* bt = a.block_tables + (int64_t)sg.seq * a.max_blocks;
    const uint8_t* kbase = a.cache + (int64_t)sg.kvh * a.page_bytes;
    const uint8_t* vbase = a.cache + (int64_t)(a.num_kv_heads + sg.kvh) * a.page_bytes;
    const int it_base = (sg.k_lo / kTileKeys) * kTileKeys;
    const int n_iter = (sg.k_hi - it_base + kDecIterKeys - 1) / kDecIterKeys;

    float m = -INFINITY;  // running max (log2 domain) of this lane's head
    float l = 0.0f;       // running sum of this lane's keys
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](IterRegs<D, MODE>& R, int it) {
      const int kA = it_base + it * kDecIterKeys;
      const int kB = kA + kTileKeys;
      const bool bok = kB < sg.k_hi;
      int32_t blkA = bt[kA / a.block_size];
      int32_t blkB = bok ? bt[kB / a.block_size] : blkA;
      // an entry outside the pool masks its tile instead of reading outside the cache
      R.oka = (uint32_t)blkA < (uint32_t)a.num_blocks;
      R.okb = bok && (uint32_t)blkB < (uint32_t)a.num_blocks;
      if (!R.oka) blkA = 0;
      if (!R.okb) blkB = blkA;
      const int rowA = kA % a.block_size, rowB = bok ? kB % a.block_size : rowA;
      const int64_t pa = (int64_t)blkA * a.block_bytes, pb = (int64_t)blkB * a.block_bytes;
      const uint8_t* ka = kbase + pa + (int64_t)(rowA + r16) * D + kg * (D / 4);
      const uint8_t* kb = kbase + pb + (int64_t)(rowB + r16) * D + kg * (D / 4);
      const uint8_t* va = vbase + pa + (int64_t)rowA * D + lane * 16;
      const uint8_t* vb = vbase + pb + (int64_t)rowB * D + lane * 16;
#pragma unroll
      for (int c = 0; c < KV4; ++c) {
        R.ka[c] = *(const uint4*)(ka + c * 16);
        R.kb[c] = *(const uint4*)(kb + c * 16);
        R.va[c] = *(const uint4*)(va + c * 1024);
        R.vb[c] = *(const uint4*)(vb + c * 1024);
      }
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
        const int64_t so = (int64_t)a.block_size * D;
        R.ksa = *(const float4*)(kbase + pa + so + 4 * (rowA + 4 * kg));
        R.ksb = *(const float4*)(kbase + pb + so + 4 * (rowB + 4 * kg));
        R.vsa = *(const float4*)(vbase + pa + so + 4 * (rowA + 4 * kg));
        R.vsb = *(const float4*)(vbase + pb + so + 4 * (rowB + 4 * kg));
      }
    };

    auto compute = [&](const IterRegs<D, MODE>& R, int it) {
      const int kA = it_base + it * kDecIterKeys;
      const int kB = kA + kTileKeys;
      // ---- S^T = K * Q^T for the two tiles
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const uint4 wa = R.ka[st / 2], wb = R.kb[st / 2];
        const uint32_t a0 = (st & 1) ? wa.z : wa.x, a1 = (st & 1) ? wa.w : wa.y;
        const uint32_t b0 = (st & 1) ? wb.z : wb.x, b1 = (st & 1) ? wb.w : wb.y;
        sa = mfma16x16x32(widen8<DT>(a0, a1), qb[st], sa);
        sb = mfma16x16x32(widen8<DT>(b0, b1), qb[st], sb);
      }
      // ---- logits of keys kA + 4kg + r (tile A) and kB + 4kg + r (tile B) for head r16
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { x[r] = sa[r] * a.logit_scale; x[4 + r] = sb[r] * a.logit_scale; }
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
        x[0] *= R.ksa.x; x[1] *= R.ksa.y; x[2] *= R.ksa.z; x[3] *= R.ksa.w;
        x[4] *= R.ksb.x; x[5] *= R.ksb.y; x[6] *= R.ksb.z; x[7] *= R.ksb.w;
      }
      if (a.softcap > 0.0f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = a.softcap * tanh_via_exp2(x[e] * a.inv_softcap);
      }
      uint32_t vmask0 = 0, vmask1 = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = (e < 4 ? kA : kB) + 4 * kg + (e & 3);
        const bool ok = key >= sg.k_lo && key < sg.k_hi && (e < 4 ? R.oka : R.okb);
        x[e] = ok ? x[e] * kLog2e : -INFINITY;
        if (ok) { if (e < 4) vmask0 |= 0xFFu << (8 * e); else vmask1 |= 0xFFu << (8 * (e - 4)); }
      }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float p[8], psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(x[e] - m_use); psum += p[e]; }
      l = l * alpha + psum;
      m = m_new;
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
        p[0] *= R.vsa.x; p[1] *= R.vsa.y; p[2] *= R.vsa.z; p[3] *= R.vsa.w;
        p[4] *= R.vsb.x; p[5] *= R.vsb.y; p[6] *= R.vsb.z; p[7] *= R.vsb.w;
      }
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)p[e];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      // ---- stage V codes: tile A rows 0..15, tile B rows 16..31 of the wave's buffer
#pragma unroll
      for (int c = 0; c < KV4; ++c) {
        *(uint4*)(vbuf + lane * 16 + c * 1024) = R.va[c];
        *(uint4*)(vbuf + kTileKeys * D + lane * 16 + c * 1024) = R.vb[c];
      }
      wave_lds_sync();
      // lane (column d = r16 of the tile, group kg) reads keys {4kg..4kg+3} of tile A and B:
      // row i of the transposed read is key (i < 4 ? 4kg + i : 16 + 4kg + i - 4).
      const int i = r16 >> 1;
      const int row = (i < 4) ? (4 * kg + i) : (kTileKeys + 4 * kg + i - 4);
      const uint8_t* rp = vbuf + row * D + (r16 & 1) * 8;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const i32x2 v = lds_read_tr8(rp + t * 16);
        const bf16x8 va = widen8<DT>((uint32_t)v.x & vmask0, (uint32_t)v.y & vmask1);
        acc[t] = mfma16x16x32(va, pb, acc[t]);
      }
      wave_lds_sync();
    };

    // software pipeline: the loads of the wave's next iteration are in flight
    // while the current one is computed
    {
      IterRegs<D, MODE> R0, R1;
      int it = wave;
      if (it < n_iter) load(R0, it);
      while (it < n_iter) {
        if (it + kDecWaves < n_iter) load(R1, it + kDecWaves);
        compute(R0, it);
        it += kDecWaves;
        if (it >= n_iter) break;
        if (it + kDecWaves < n_iter) load(R0, it + kDecWaves);
        compute(R1, it);
        it += kDecWaves;
      }
    }

    // ---- merge the four waves: l over the lanes of a head, then across waves in LDS
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    __syncthreads();  // every wave is done with its V staging buffer
    float* mg = (float*)smem;  // [wave-1][head][D + 2]
    if (wave > 0) {
      float* dst = mg + ((wave - 1) * kMaxHeadsPerUnit + r16) * (D + 2);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[t * 16 + 4 * kg + r] = acc[t][r];
      if (kg == 0) { dst[D] = m; dst[D + 1] = l; }
    }
    __syncthreads();
    if (wave == 0) {
      float mw[kDecWaves], lw[kDecWaves];
      mw[0] = m; lw[0] = l;
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) {
        const float* src = mg + ((w - 1) * kMaxHeadsPerUnit + r16) * (D + 2);
        mw[w] = src[D]; lw[w] = src[D + 1];
      }
      float M = mw[0];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, mw[w]);
      const float M_use = M == -INFINITY ? 0.0f : M;
      float f[kDecWaves], L = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) { f[w] = fast_exp2(mw[w] - M_use); L += f[w] * lw[w]; }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t] *= f[0];
#pragma unroll
        for (int w = 1; w < kDecWaves; ++w) {
          const float* src = mg + ((w - 1) * kMaxHeadsPerUnit + r16) * (D + 2) + t * 16 + 4 * kg;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][r] += f[w] * src[r];
        }
      }
      if (head_ok) {
        if (sg.part < 0) {
          const float norm = a.v_scale / L;
          uint16_t* op = a.out + ((int64_t)sg.q_tok * a.num_q_heads + hq) * D;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            uint2 w;
            w.x = (uint32_t)f32_to_bf16_rne(acc[t][0] * norm) | ((uint32_t)f32_to_bf16_rne(acc[t][1] * norm) << 16);
            w.y = (uint32_t)f32_to_bf16_rne(acc[t][2] * norm) | ((uint32_t)f32_to_bf16_rne(acc[t][3] * norm) << 16);
            *(uint2*)(op + t * 16 + 4 * kg) = w;
          }
        } else {
          // partial slot: O at [part][head][D], (m, l) at [part][head][2] after all O slots
          float* pp = a.scratch + ((int64_t)sg.part * a.group_heads + r16) * D;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            float4 w = make_float4(acc[t][0] * a.v_scale, acc[t][1] * a.v_scale, acc[t][2] * a.v_scale,
                                   acc[t][3] * a.v_scale);
            *(float4*)(pp + t * 16 + 4 * kg) = w;
          }
          if (kg == 0) {
            float* ml = a.scratch + (int64_t)a.num_parts * a.group_heads * D + ((int64_t)sg.part * a.group_heads + r16) * 2;
            ml[0] = M;
            ml[1] = L;
          }
        }
      }
    }
    __syncthreads();  // the merge area is reused as staging by the next segment
  }
}

// Split-KV merge: one wave per (item, head). M = max_s m_s;
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const CombItem* items, const float* scratch, uint16_t* out,
                                                     int32_t num_q_heads, int32_t group, int32_t group_heads,
                                                     int32_t num_parts) {
  const CombItem it = items[blockIdx.x];
  const int h = blockIdx.y;
  if (h >= it.nheads) return;
  const int lane = threadIdx.x;
  const float* ml = scratch + (int64_t)num_parts * group_heads * D;
  float M = -INFINITY;
  for (int s = 0; s < it.num_parts; ++s) M = fmaxf(M, ml[((int64_t)(it.first_part + s) * group_heads + h) * 2]);
  const float M_use = M == -INFINITY ? 0.0f : M;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] = 0.0f;
  float L = 0.0f;
  for (int s = 0; s < it.num_parts; ++s) {
    const int64_t slot = (int64_t)(it.first_part + s) * group_heads + h;
    const float* pp = scratch + slot * D;
    const float f = fast_exp2(ml[slot * 2] - M_use);
    L += f * ml[slot * 2 + 1];
#pragma unroll
    for (int j = 0; j < PER; ++j) o[j] += f * pp[lane + 64 * j];
  }
  const float inv = 1.0f / L;
  uint16_t* op = out + ((int64_t)it.q_tok * num_q_heads + it.kvh * group + it.head0 + h) * D;
#pragma unroll
  for (int j = 0; j < PER; ++j) op[lane + 64 * j] = f32_to_bf16_rne(o[j] * inv);
}

template <int D, int DT, int MODE>
static int launch_dec(const AttnArgs& a, hipStream_t st) {
  const SchedHeader& h = *a.hdr;
  DecArgs d;
  d.cache = a.cache;
  d.q = a.q;
  d.block_tables = a.block_tables;
  d.segs = (const DecSeg*)(a.meta_dev + h.off_dec_segs);
  d.wg_start = (const int32_t*)(a.meta_dev + h.off_dec_wg_start);
  d.scratch = a.scratch;
  d.out = a.out;
  d.page_bytes = a.page_bytes;
  d.block_bytes = a.block_bytes;
  d.block_size = a.block_size;
  d.num_kv_heads = a.num_kv_heads;
  d.num_q_heads = a.num_q_heads;
  d.group = a.group;
  d.max_blocks = a.max_blocks_per_seq;
  d.group_heads = h.group_heads;
  d.num_blocks = h.num_blocks;
  d.num_parts = h.num_parts;
  d.logit_scale = MODE == AQP_SCALE_PER_TENSOR ? a.sm_scale * a.k_scale : a.sm_scale;
  d.softcap = a.softcap;
  d.inv_softcap = a.softcap > 0.0f ? 1.0f / a.softcap : 0.0f;
  d.v_scale = MODE == AQP_SCALE_PER_TENSOR ? a.v_scale : 1.0f;
  hipLaunchKernelGGL((decode_kernel<D, DT, MODE>), dim3(h.num_dec_wgs), dim3(256), h.dec_lds_bytes, st, d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("aqp_paged_attention: decode launch failed: %s", hipGetErrorString(e));
    return AQP_ERR_HIP;
  }
  return AQP_OK;
}

template <int DT, int MODE>
static int dec_d(const AttnArgs& a, hipStream_t st) {
  switch (a.head_dim) {
    case 64: return launch_dec<64, DT, MODE>(a, st);
    case 128: return launch_dec<128, DT, MODE>(a, st);
    case 256: return launch_dec<256, DT, MODE>(a, st);
  }
  set_error("aqp_paged_attention: unsupported head_dim %d", a.head_dim);
  return AQP_ERR_UNSUPPORTED;
}

int launch_decode(int dtype, int mode, const AttnArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E4M3) return dec_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E5M2) return dec_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_INT8) return dec_d<AQP_KV_INT8, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E4M3) return dec_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  set_error("aqp_paged_attention: dtype %d with scale mode %d is not built", dtype, mode);
  return AQP_ERR_UNSUPPORTED;
}

int launch_combine(const AttnArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const SchedHeader& h = *a.hdr;
  const CombItem* items = (const CombItem*)(a.meta_dev + h.off_comb);
  dim3 grid(h.num_comb, h.group_heads);
  switch (a.head_dim) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(64), 0, st, items, a.scratch, a.out, a.num_q_heads, a.group, h.group_heads, h.num_parts); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(64), 0, st, items, a.scratch, a.out, a.num_q_heads, a.group, h.group_heads, h.num_parts); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(64), 0, st, items, a.scratch, a.out, a.num_q_heads, a.group, h.group_heads, h.num_parts); break;
    default: set_error("aqp_paged_attention: unsupported head_dim"); return AQP_ERR_UNSUPPORTED;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("aqp_paged_attention: combine launch failed: %s", hipGetErrorString(e));
    return AQP_ERR_HIP;
  }
  return AQP_OK;
}

}  // namespace aqp
