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
//  * a wave takes 16-key tiles w, w+4, ... of the segment;
//  * K: each lane loads D/4 contiguous code bytes of one key straight from HBM
//    (16 keys x D bytes of a page per tile); the codes are widened to bf16 in
//    registers and fed to v_mfma_f32_16x16x32_bf16 as S^T = K * Q^T with the
//    group's q heads as the 16 MFMA columns;
//  * scale folding: per tensor, k_scale goes into the logit scale and v_scale
//    into the final normalisation; per token-head, each key's scale multiplies
//    its logit and each value's scale its probability;
//  * softmax: running max / sum in the exp2 domain, the max reduced across the
//    four lanes that share a head with two xor shuffles;
//  * V: the tile's codes are staged in the wave's own LDS buffer and read back
//    with ds_read_b64_tr_b8, which hands each lane 4 keys of one head-dim column
//    for two column tiles at once: the key-contiguous operand that
//    O^T = V^T * P^T on v_mfma_f32_16x16x16_bf16 needs, so the probabilities
//    stay in the registers the QK^T product left them in;
//  * the four waves' (m, l, O) are merged in LDS; the result is either the
//    output row (bf16) or a partial slot for the split-KV merge kernel.
#include "device_common.h"

// Decode waves per SIMD the register allocation targets for head_dim <= 128
// (head_dim 256 targets 2).
#ifndef AQP_DECODE_WAVES_PER_EU
#define AQP_DECODE_WAVES_PER_EU 3
#endif

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
struct TileRegs {
  static constexpr int KV4 = D / 64;  // uint4 per lane per 16-key tile (D/4 bytes)
  uint4 k[KV4];                       // K codes: one key row slice per lane (MFMA A layout)
  uint4 v[KV4];                       // V codes: coalesced slices of the tile
  float4 ks, vs;                      // per token-head scales of the lane's 4 keys
  bool ok;                            // the tile's block id is inside the pool
};

template <int D, int DT, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 128 ? AQP_DECODE_WAVES_PER_EU : 2))) void decode_kernel(DecArgs a) {
  constexpr int KV4 = D / 64;
  constexpr int NT = D / 16;   // 16-wide head-dim tiles of the output
  constexpr int QS = D / 32;   // 32-deep MFMA steps of QK^T
  constexpr int VROW = D + kDecVRowPad;  // staged V row stride in LDS
  constexpr int STEP = kDecWaves * kDecIterKeys;  // keys between a wave's consecutive tiles
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  uint8_t* vbuf = smem + wave * (kDecIterKeys * VROW);
  // where this lane's V chunks go in the padded staging rows
  int vdst[KV4];
#pragma unroll
  for (int c = 0; c < KV4; ++c) {
    const int o = lane * 16 + c * 1024;
    vdst[c] = (o / D) * VROW + (o % D);
  }
  // transposed-read address of this lane: rows i = 0..3 and 4..7 are keys 4kg + (i & 3), the
  // second four 16 columns further, so one read yields the operands of two head-dim tiles
  const int tr_i = r16 >> 1;
  const int tr_off = (4 * kg + (tr_i & 3)) * VROW + (tr_i >> 2) * 16 + (r16 & 1) * 8;
  const int s_begin = as_const(a.wg_start)[blockIdx.x], s_end = as_const(a.wg_start)[blockIdx.x + 1];
  // without a soft-cap, log2(e) folds into the logit scale
  const float xscale = a.softcap > 0.0f ? a.logit_scale : a.logit_scale * kLog2e;

  for (int si = s_begin; si < s_end; ++si) {
    const DecSeg sg = load_const(as_const(a.segs) + si);
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
    const cptr<int32_t> bt = as_const(a.block_tables) + (int64_t)sg.seq * a.max_blocks;
    const uint8_t* kbase = a.cache + (int64_t)sg.kvh * a.page_bytes;
    const uint8_t* vbase = a.cache + (int64_t)(a.num_kv_heads + sg.kvh) * a.page_bytes;
    const int it_base = (sg.k_lo / kTileKeys) * kTileKeys;
    const int n_iter = (sg.k_hi - it_base + kDecIterKeys - 1) / kDecIterKeys;

    float m = -INFINITY;  // reference max (log2 domain) of this lane's head
    float l = 0.0f;       // sum of this lane's probabilities relative to m
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // position of a tile: logical block index and first row, advanced incrementally
    struct Pos { int k0, bi, r0; };
    auto advance = [&](Pos p) {
      p.k0 += STEP;
      p.r0 += STEP;
      while (p.r0 >= a.block_size) { p.r0 -= a.block_size; ++p.bi; }
      return p;
    };

    auto load = [&](TileRegs<D, MODE>& R, const Pos& p) {
      int32_t blk = bt[p.bi];
      // an entry outside the pool masks its tile instead of reading outside the cache
      R.ok = (uint32_t)blk < (uint32_t)a.num_blocks;
      if (!R.ok) blk = 0;
      const int64_t pb = (int64_t)blk * a.block_bytes;
      const uint8_t* kp = kbase + pb + (int64_t)(p.r0 + r16) * D + kg * (D / 4);
      const uint8_t* vp = vbase + pb + (int64_t)p.r0 * D + lane * 16;
#pragma unroll
      for (int c = 0; c < KV4; ++c) {
        R.k[c] = *(const uint4*)(kp + c * 16);
        R.v[c] = *(const uint4*)(vp + c * 1024);
      }
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
        const int64_t so = (int64_t)a.block_size * D + 4 * (p.r0 + 4 * kg);
        R.ks = *(const float4*)(kbase + pb + so);
        R.vs = *(const float4*)(vbase + pb + so);
      }
    };

    auto compute = [&](const TileRegs<D, MODE>& R, const Pos& p) {
      // ---- S^T = K * Q^T: lane holds keys k0 + 4kg + r of head r16
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const uint4 w = R.k[st / 2];
        const uint32_t w0 = (st & 1) ? w.z : w.x, w1 = (st & 1) ? w.w : w.y;
        s = mfma16x16x32(widen8<DT>(w0, w1), qb[st], s);
      }
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = s[r] * xscale;
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
        x[0] *= R.ks.x; x[1] *= R.ks.y; x[2] *= R.ks.z; x[3] *= R.ks.w;
      }
      if (a.softcap > 0.0f) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = a.softcap * kLog2e * tanh_via_exp2(x[r] * a.inv_softcap);
      }
      // masking is needed only on the segment's edge tiles (and tiles of an invalid block)
      const bool full = R.ok && p.k0 >= sg.k_lo && p.k0 + kTileKeys <= sg.k_hi;
      uint32_t vmask = 0xFFFFFFFFu;
      if (!full) {
        vmask = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = p.k0 + 4 * kg + r;
          const bool ok = R.ok && key >= sg.k_lo && key < sg.k_hi;
          x[r] = ok ? x[r] : -INFINITY;
          if (ok) vmask |= 0xFFu << (8 * r);
        }
      }
      // rows outside the range may hold unwritten bytes: their V codes are masked to zero and
      // (per token-head) their scale is replaced, so no NaN pattern reaches the sums
      const float mx = max_over_rows(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      // lazy rescaling: the reference max moves (and O, l are rescaled) only when some head's
      // max exceeds it by more than 2^8, so probabilities stay <= 256 and the common case
      // leaves the accumulators alone
      if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.0f : m_new));
        l *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] *= alpha;
        m = m_new;
      }
      const float m_use = m == -INFINITY ? 0.0f : m;
      float p4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p4[r] = fast_exp2(x[r] - m_use);
      l += (p4[0] + p4[1]) + (p4[2] + p4[3]);
      if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
        float4 vs = R.vs;
        if (!full) {
          vs.x = (vmask & 0xFFu) ? vs.x : 0.0f;
          vs.y = (vmask & 0xFF00u) ? vs.y : 0.0f;
          vs.z = (vmask & 0xFF0000u) ? vs.z : 0.0f;
          vs.w = (vmask & 0xFF000000u) ? vs.w : 0.0f;
        }
        p4[0] *= vs.x; p4[1] *= vs.y; p4[2] *= vs.z; p4[3] *= vs.w;
      }
      bf16x4 pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[r] = (__bf16)p4[r];
      // ---- stage the V tile, read it transposed: O^T[d][head] += V^T[d][keys] P^T[keys][head]
#pragma unroll
      for (int c = 0; c < KV4; ++c) *(uint4*)(vbuf + vdst[c]) = R.v[c];
      wave_lds_sync();
#pragma unroll
      for (int t2 = 0; t2 < NT / 2; ++t2) {
        const i32x2 v = lds_read_tr8(vbuf + tr_off + t2 * 32);
        acc[2 * t2] = mfma16x16x16(widen4v<DT>((uint32_t)v.x & vmask), pb, acc[2 * t2]);
        acc[2 * t2 + 1] = mfma16x16x16(widen4v<DT>((uint32_t)v.y & vmask), pb, acc[2 * t2 + 1]);
      }
      wave_lds_sync();
    };

    // software pipeline: the loads of the wave's next tile are in flight while
    // the current one is computed
    if (wave < n_iter) {
      Pos p0, p1;
      p0.k0 = it_base + wave * kDecIterKeys;
      p0.bi = p0.k0 / a.block_size;
      p0.r0 = p0.k0 - p0.bi * a.block_size;
      TileRegs<D, MODE> R0, R1;
      load(R0, p0);
      int it = wave;
      while (true) {
        p1 = advance(p0);
        const bool more1 = it + kDecWaves < n_iter;
        if (more1) load(R1, p1);
        compute(R0, p0);
        if (!more1) break;
        it += kDecWaves;
        p0 = advance(p1);
        const bool more0 = it + kDecWaves < n_iter;
        if (more0) load(R0, p0);
        compute(R1, p1);
        if (!more0) break;
        it += kDecWaves;
      }
    }

    // ---- merge the four waves: l over the lanes of a head, then across waves in LDS
    l = sum_over_rows(l);
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
  const CombItem it = load_const(as_const(items) + blockIdx.x);
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
