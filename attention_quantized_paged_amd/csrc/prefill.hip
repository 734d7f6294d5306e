// Prefill attention (several query tokens per sequence, causal or not) over
// the quantised paged cache.
//
// Same method as decode (dequantise fused into the QK^T and PV tile products,
// online softmax, folded scales: the "CPU backend adds FP8 KV-cache
// quantisation" page, vllm PR 39445, Implementation item 2; the large-prefill
// case the "Fix CPU FP8 attention scheduler scratch sizing" page, vllm PR
// 50194, stresses with block_size 2176 and head_size 256).
//
// gfx950 mapping: one work-group of 4 waves per schedule item (a run of query
// tokens of one sequence times the q heads of one KV head = up to 128 query
// rows, token-major, so all rows share the K/V tiles). Each step stages the
// codes of 32 keys of K and V (and their per-token-head scales) in LDS,
// double-buffered, with one cooperative 16-byte load per chunk; every wave
// then runs, for its 32 rows (two 16-row MFMA column blocks):
//   S^T = K * Q^T   (A = K codes read from LDS and widened to bf16; B = Q^T in
//                    registers for the whole item)
//   online softmax per row (4 keys per lane per 16-key tile, max over the
//                    4 lanes of a row with xor shuffles)
//   O^T += V^T * P^T (A = V codes via ds_read_b64_tr_b8, B = the
//                    probabilities exactly where S^T left them)
// The 32-key step is the kernel's compile-time tile; the schedule records it
// and the element sizes the LDS was sized with, and the launcher checks both.
#include "device_common.h"

namespace aqp {

struct PfArgs {
  const uint8_t* cache;
  const uint16_t* q;
  const int32_t* block_tables;
  const PfItem* items;
  uint16_t* out;
  int64_t page_bytes, block_bytes;
  int32_t block_size, num_kv_heads, num_q_heads, group, max_blocks, num_blocks;
  int32_t causal, window;
  float logit_scale;  // sm_scale * k_scale (per tensor) or sm_scale (per token-head)
  float softcap, inv_softcap;
  float v_scale;
};

template <int D, int DT, int MODE>
__global__ __launch_bounds__(256) void prefill_kernel(PfArgs a) {
  constexpr int NT = D / 16;
  constexpr int QS = D / 32;
  constexpr int KT = kPfKvTile;                // keys per step
  constexpr int CHUNKS = KT * D / 16;          // 16-byte chunks per K (or V) step
  constexpr int CPT = (CHUNKS + 255) / 256;    // chunks per thread
  constexpr int BUF = 2 * KT * D + 2 * KT * 4; // bytes per LDS buffer: K, V codes, K, V scales
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const PfItem it = a.items[blockIdx.x];
  const int G = a.group;
  const int ntok = it.q_hi - it.q_lo;
  const int32_t* bt = a.block_tables + (int64_t)it.seq * a.max_blocks;
  const uint8_t* kbase = a.cache + (int64_t)it.kvh * a.page_bytes;
  const uint8_t* vbase = a.cache + (int64_t)(a.num_kv_heads + it.kvh) * a.page_bytes;

  // ---- rows of this lane (as MFMA column r16 of row tiles 0, 1)
  int lo_r[2], hi_r[2];
  bool row_ok[2];
  int64_t orow[2];
  bf16x8 qb[2][QS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = wave * kPfRowsPerWave + rt * 16 + r16;
    const int tl = row / G, g = row - (row / G) * G;
    row_ok[rt] = tl < ntok;
    const int t = it.q_lo + (row_ok[rt] ? tl : 0);
    const int p = it.L - it.ql + t;
    hi_r[rt] = a.causal ? p + 1 : it.L;
    lo_r[rt] = (a.window > 0 && p - a.window + 1 > 0) ? p - a.window + 1 : 0;
    if (!row_ok[rt]) { lo_r[rt] = 0; hi_r[rt] = 0; }
    orow[rt] = ((int64_t)(it.q_start + t) * a.num_q_heads + it.kvh * G + g) * D;
    const uint16_t* qp = a.q + orow[rt] + kg * (D / 4);
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      uint4 u = *(const uint4*)(qp + st * 8);
      if (!row_ok[rt]) u = make_uint4(0, 0, 0, 0);
      qb[rt][st] = __builtin_bit_cast(bf16x8, u);
    }
  }
  // ---- key range of the whole item: first token's window start .. last token's end
  const int p_first = it.L - it.ql + it.q_lo;
  const int k_first = (a.window > 0 && p_first - a.window + 1 > 0) ? p_first - a.window + 1 : 0;
  const int k_begin = (k_first / kTileKeys) * kTileKeys;
  const int k_end = it.k_hi_max;
  const int n_steps = (k_end - k_begin + KT - 1) / KT;

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4 acc[2][NT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // cooperative staging registers
  uint4 kreg[CPT], vreg[CPT];
  float sreg = 0.0f;
  auto gload = [&](int step) {
    const int kb0 = k_begin + step * KT;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * 256;
      kreg[c] = make_uint4(0, 0, 0, 0);
      vreg[c] = make_uint4(0, 0, 0, 0);
      if (ch < CHUNKS) {
        const int key = ch / (D / 16), col = (ch % (D / 16)) * 16;
        const int j = kb0 + key;
        if (j < it.L) {
          const int32_t blk = bt[j / a.block_size];
          if ((uint32_t)blk < (uint32_t)a.num_blocks) {
            const int64_t off = (int64_t)blk * a.block_bytes + (int64_t)(j % a.block_size) * D + col;
            kreg[c] = *(const uint4*)(kbase + off);
            vreg[c] = *(const uint4*)(vbase + off);
          }
        }
      }
    }
    if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
      sreg = 0.0f;
      if (tid < 2 * KT) {
        const int j = kb0 + (tid % KT);
        if (j < it.L) {
          const int32_t blk = bt[j / a.block_size];
          if ((uint32_t)blk < (uint32_t)a.num_blocks) {
            const uint8_t* base = tid < KT ? kbase : vbase;
            sreg = *(const float*)(base + (int64_t)blk * a.block_bytes + (int64_t)a.block_size * D + 4 * (j % a.block_size));
          }
        }
      }
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* b = smem + buf * BUF;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * 256;
      if (ch < CHUNKS) {
        *(uint4*)(b + ch * 16) = kreg[c];
        *(uint4*)(b + KT * D + ch * 16) = vreg[c];
      }
    }
    if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) {
      if (tid < 2 * KT) *(float*)(b + 2 * KT * D + 4 * tid) = sreg;
    }
  };

  if (n_steps > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    if (step + 1 < n_steps) gload(step + 1);
    const uint8_t* kl = smem + buf * BUF;
    const uint8_t* vl = kl + KT * D;
    const float* ksl = (const float*)(kl + 2 * KT * D);
    const float* vsl = ksl + KT;
    const int kb0 = k_begin + step * KT;
    // ---- S^T = K Q^T: [key tile kt][row tile rt]
    f32x4 s[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) s[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* kp = kl + (kt * 16 + r16) * D + kg * (D / 4);
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const uint2 w = *(const uint2*)(kp + st * 8);
        const bf16x8 ka = widen8<DT>(w.x, w.y);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) s[kt][rt] = mfma16x16x32(ka, qb[rt][st], s[kt][rt]);
      }
    }
    // ---- online softmax per row tile
    bf16x8 pb[2];
    float alpha[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kt = e >> 2, r = e & 3;
        float v = s[kt][rt][r] * a.logit_scale;
        if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) v *= ksl[kt * 16 + 4 * kg + r];
        if (a.softcap > 0.0f) v = a.softcap * tanh_via_exp2(v * a.inv_softcap);
        const int j = kb0 + kt * 16 + 4 * kg + r;
        x[e] = (j >= lo_r[rt] && j < hi_r[rt]) ? v * kLog2e : -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float m_new = fmaxf(m[rt], mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      alpha[rt] = fast_exp2(m[rt] - m_use);
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pe = fast_exp2(x[e] - m_use);
        psum += pe;
        if constexpr (MODE == AQP_SCALE_PER_TOKEN_HEAD) pe *= vsl[(e >> 2) * 16 + 4 * kg + (e & 3)];
        pb[rt][e] = (__bf16)pe;
      }
      l[rt] = l[rt] * alpha[rt] + psum;
      m[rt] = m_new;
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[rt][t] *= alpha[rt];
    // ---- O^T += V^T P^T; transposed row i of the read is key (i < 4 ? 4kg + i : 16 + 4kg + i - 4)
    {
      const int i = r16 >> 1;
      const int row = (i < 4) ? (4 * kg + i) : (16 + 4 * kg + i - 4);
      const uint8_t* rp = vl + row * D + (r16 & 1) * 8;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const i32x2 v = lds_read_tr8(rp + t * 16);
        const bf16x8 va = widen8<DT>((uint32_t)v.x, (uint32_t)v.y);
        acc[0][t] = mfma16x16x32(va, pb[0], acc[0][t]);
        acc[1][t] = mfma16x16x32(va, pb[1], acc[1][t]);
      }
    }
    if (step + 1 < n_steps) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and write the rows
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float lt = l[rt];
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    if (!row_ok[rt]) continue;
    const float norm = a.v_scale / lt;
    uint16_t* op = a.out + orow[rt];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16_rne(acc[rt][t][0] * norm) | ((uint32_t)f32_to_bf16_rne(acc[rt][t][1] * norm) << 16);
      w.y = (uint32_t)f32_to_bf16_rne(acc[rt][t][2] * norm) | ((uint32_t)f32_to_bf16_rne(acc[rt][t][3] * norm) << 16);
      *(uint2*)(op + t * 16 + 4 * kg) = w;
    }
  }
}

template <int D, int DT, int MODE>
static int launch_pf(const AttnArgs& a, hipStream_t st) {
  const SchedHeader& h = *a.hdr;
  PfArgs p;
  p.cache = a.cache;
  p.q = a.q;
  p.block_tables = a.block_tables;
  p.items = (const PfItem*)(a.meta_dev + h.off_pf_items);
  p.out = a.out;
  p.page_bytes = a.page_bytes;
  p.block_bytes = a.block_bytes;
  p.block_size = a.block_size;
  p.num_kv_heads = a.num_kv_heads;
  p.num_q_heads = a.num_q_heads;
  p.group = a.group;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = h.num_blocks;
  p.causal = a.causal;
  p.window = a.window;
  p.logit_scale = MODE == AQP_SCALE_PER_TENSOR ? a.sm_scale * a.k_scale : a.sm_scale;
  p.softcap = a.softcap;
  p.inv_softcap = a.softcap > 0.0f ? 1.0f / a.softcap : 0.0f;
  p.v_scale = MODE == AQP_SCALE_PER_TENSOR ? a.v_scale : 1.0f;
  hipLaunchKernelGGL((prefill_kernel<D, DT, MODE>), dim3(h.num_pf_items), dim3(256), h.pf_lds_bytes, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("aqp_paged_attention: prefill launch failed: %s", hipGetErrorString(e));
    return AQP_ERR_HIP;
  }
  return AQP_OK;
}

template <int DT, int MODE>
static int pf_d(const AttnArgs& a, hipStream_t st) {
  switch (a.head_dim) {
    case 64: return launch_pf<64, DT, MODE>(a, st);
    case 128: return launch_pf<128, DT, MODE>(a, st);
    case 256: return launch_pf<256, DT, MODE>(a, st);
  }
  set_error("aqp_paged_attention: unsupported head_dim %d", a.head_dim);
  return AQP_ERR_UNSUPPORTED;
}

int launch_prefill(int dtype, int mode, const AttnArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E4M3) return pf_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E5M2) return pf_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_INT8) return pf_d<AQP_KV_INT8, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E4M3) return pf_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  set_error("aqp_paged_attention: dtype %d with scale mode %d is not built", dtype, mode);
  return AQP_ERR_UNSUPPORTED;
}

}  // namespace aqp
