// Prefill attention (several query tokens per sequence, causal or not) over
// the quantised paged cache.
//
// Same method as decode (dequantise fused into the QK^T and PV tile products,
// online softmax, folded scales: the "CPU backend adds FP8 KV-cache
// quantisation" page, vllm PR 39445, Implementation item 2; the large-prefill
// case the "Fix CPU FP8 attention scheduler scratch sizing" page, vllm PR
// 50194, stresses with block_size 2176 and head_size 256).
//
// gfx950 mapping: one work-group per schedule item (a run of query tokens of
// one sequence times a run of the q heads of one KV head = up to 128 query rows,
// token-major, so all rows share the K/V tiles); 4 waves of 32 rows, or 8 waves
// of 16 rows at head_dim 256 (two waves per SIMD). Each step copies
// the codes of 32 keys of K and V (and their per-token-head scales) straight
// from HBM into a 4-stage LDS ring (global_load_lds, XOR-swizzled 16-byte
// chunks); every wave then runs, for its rows (16-row MFMA column blocks):
//   S^T = K * Q^T   (A = K codes read from LDS and widened to bf16; B = Q^T in
//                    registers for the whole item)
//   online softmax per row (4 keys per lane per 16-key tile, max over the
//                    4 lanes of a row with lane permutes)
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

// 16-byte chunk swizzle of a staged row: chunk c of row `row` is stored at chunk
// c ^ swz(row). Rows are D bytes; 256 bytes span all LDS banks, so rows that share banks
// (same row / (256 / D) residue) get different chunk offsets, and the second 16-key tile gets
// the upper half of the offsets. This keeps the K-operand reads (16 rows, one chunk) and the
// transposed V reads (8 rows of two tiles, one chunk) free of bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int row) {
  constexpr int CPR = D / 16;                  // chunks per row
  constexpr int RPL = D >= 256 ? 1 : 256 / D;  // rows per 256 bytes
  return ((row / RPL) % CPR) ^ (((row >> 4) & 1) * (CPR / 2));
}

template <int D, int DT, int MODE, bool CAP>
__global__ __launch_bounds__(pf_waves(D) * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2))) void prefill_kernel(PfArgs a) {
  constexpr int NT = D / 16;
  constexpr int QS = D / 32;
  constexpr int WAVES = pf_waves(D);
  constexpr int RT = kPfRows / (16 * WAVES);      // 16-row MFMA column blocks per wave
  constexpr int RPW = 16 * RT;                    // query rows per wave
  constexpr int KT = kPfKvTile;                   // keys per step (two 16-key tiles)
  constexpr int NS = kPfStages;                   // LDS ring stages
  constexpr int CPR = D / 16;                     // 16-byte chunks per row
  constexpr int STAGE = 2 * KT * D + 2 * KT * 4;  // K codes, V codes, K scales, V scales
  constexpr int KV_INSTR = KT * CPR / 64;         // 1 KB copies per K (or V) step
  constexpr int IPW = 2 * KV_INSTR / WAVES;       // K+V copies per wave per step
  static_assert(IPW >= 1 && (2 * KV_INSTR) % WAVES == 0, "copies must split evenly over the waves");
  constexpr int PTH = MODE == AQP_SCALE_PER_TOKEN_HEAD ? 1 : 0;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const PfItem it = load_const(as_const(a.items) + blockIdx.x);
  const int G = a.group;
  const int nh = it.nheads;  // q heads per token in this item
  const int ntok = it.q_hi - it.q_lo;
  const cptr<int32_t> bt = as_const(a.block_tables) + (int64_t)it.seq * a.max_blocks;
  const uint8_t* kbase = a.cache + (int64_t)it.kvh * a.page_bytes;
  const uint8_t* vbase = a.cache + (int64_t)(a.num_kv_heads + it.kvh) * a.page_bytes;
  const uint32_t lds0 = lds_addr(smem);
  // copies this wave issues per step: its share of K/V, plus the scale copy on the last wave
  const int ipw_me = IPW + ((PTH && wave == WAVES - 1) ? 1 : 0);

  // ---- rows of this lane (as MFMA column r16 of the wave's row tiles)
  int lo_r[RT], hi_r[RT];
  bool row_ok[RT];
  int64_t orow[RT];
  bf16x8 qb[RT][QS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = wave * RPW + rt * 16 + r16;
    const int tl = row / nh, g = it.head0 + row - (row / nh) * nh;
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
  // the wave's rows cover tokens [tw0, tw1]: keys in [vis_lo, vis_hi) are visible to all of them
  const int tw0 = min(ntok - 1, (wave * RPW) / nh);
  const int tw1 = min(ntok - 1, (wave * RPW + RPW - 1) / nh);
  const bool wave_rows_full = (wave * RPW + RPW - 1) / nh < ntok;
  const int pw0 = it.L - it.ql + it.q_lo + tw0, pw1 = it.L - it.ql + it.q_lo + tw1;
  const int vis_hi = a.causal ? pw0 + 1 : it.L;
  const int vis_lo = (a.window > 0 && pw1 - a.window + 1 > 0) ? pw1 - a.window + 1 : 0;
  // ---- key range of the whole item: first token's window start .. last token's end
  const int p_first = it.L - it.ql + it.q_lo;
  const int k_first = (a.window > 0 && p_first - a.window + 1 > 0) ? p_first - a.window + 1 : 0;
  const int k_begin = (k_first / kTileKeys) * kTileKeys;
  const int k_end = it.k_hi_max;
  const int n_steps = (k_end - k_begin + KT - 1) / KT;
  const float xscale = CAP ? a.logit_scale : a.logit_scale * kLog2e;
  const int last_tile = ((it.L - 1) / kTileKeys) * kTileKeys;  // first key of the tile holding key L-1

  float m[RT], l[RT];
  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.0f;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- issue the copies of one step into its ring stage. Copy ii (0 .. 2*KV_INSTR-1) fills
  // 64 chunks of K (ii < KV_INSTR) or V; lane l takes LDS chunk q = 64*(ii % KV_INSTR) + l,
  // row q / CPR, stored chunk q % CPR, which holds logical chunk (q % CPR) ^ swz(row). The 64
  // chunks lie in one 16-key tile. Keys at or past L (never visible) read key L-1's row so that
  // only finite codes reach LDS.
  auto issue = [&](int step) {
    const int kb0 = k_begin + step * KT;
    const uint32_t sbase = lds0 + (uint32_t)((step % NS) * STAGE);
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int ii = wave + WAVES * j;
      const int kv = ii / KV_INSTR;
      const int q0 = 64 * (ii % KV_INSTR);
      const int q = q0 + lane;
      const int row = q / CPR;
      const int lc = (q % CPR) ^ swz<D>(row);
      // tile of this copy (uniform), clamped to the tile of key L-1
      const int tile_k0 = min(kb0 + ((q0 / CPR) & ~15), last_tile);
      const int tbi = tile_k0 / a.block_size;
      const int tr0 = tile_k0 - tbi * a.block_size;
      int32_t blk = bt[tbi];
      if ((uint32_t)blk >= (uint32_t)a.num_blocks) blk = 0;  // invalid table entry: stay in the pool
      const int key = min(kb0 + row, it.L - 1);
      const uint8_t* src = (kv ? vbase : kbase) + (int64_t)blk * a.block_bytes +
                           (int64_t)(tr0 + (key - tile_k0)) * D + lc * 16;
      dma16_to_lds(src, sbase + (uint32_t)(kv * KT * D + q0 * 16));
    }
    if constexpr (PTH) {
      if (wave == WAVES - 1) {
        // 16 lanes x 16 bytes: [K scales of the 32 keys][V scales], 4 scales per lane
        const int tl = (lane >> 2) & 1, part = lane & 3, kv = lane >> 3;
        const int t0 = min(kb0, last_tile), t1 = min(kb0 + 16, last_tile);
        const int bi0 = t0 / a.block_size, bi1 = t1 / a.block_size;
        int32_t b0 = bt[bi0], b1 = bt[bi1];
        if ((uint32_t)b0 >= (uint32_t)a.num_blocks) b0 = 0;
        if ((uint32_t)b1 >= (uint32_t)a.num_blocks) b1 = 0;
        const int tk0 = tl ? t1 : t0;
        const int32_t blk = tl ? b1 : b0;
        const int r0 = tk0 - (tl ? bi1 : bi0) * a.block_size;
        const uint8_t* src = (kv ? vbase : kbase) + (int64_t)blk * a.block_bytes + (int64_t)a.block_size * D +
                             4 * (r0 + 4 * part);
        if (lane < 16) dma16_to_lds(src, sbase + (uint32_t)(2 * KT * D));
      }
    }
  };

  // transposed V read: row i of lane group kg is key (i < 4 ? 4kg + i : 16 + 4kg + i - 4)
  const int tr_i = r16 >> 1;
  const int tr_row = (tr_i < 4) ? (4 * kg + tr_i) : (16 + 4 * kg + tr_i - 4);
  const int tr_swz = swz<D>(tr_row);

  // ---- S^T = K Q^T of one step: [key tile kt][row tile rt]. The operand reads of the whole step
  // are issued before any use, so the LDS latency of one overlaps the work on the others.
  auto qk = [&](int step, f32x4 (&s)[2][RT]) {
    const uint8_t* kl = smem + (step % NS) * STAGE;
    uint2 kw[2][QS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int krow = kt * 16 + r16;
      const uint8_t* kp = kl + krow * D;
      const int ksw = swz<D>(krow);
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const int dbyte = kg * (D / 4) + st * 8;
        kw[kt][st] = *(const uint2*)(kp + ((((dbyte >> 4) ^ ksw) << 4) | (dbyte & 8)));
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const bf16x8 ka = widen8<DT>(kw[kt][st].x, kw[kt][st].y);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) s[kt][rt] = mfma16x16x32(ka, qb[rt][st], s[kt][rt]);
      }
    }
  };

  // ---- online softmax of one step's S (lazy rescaling as in decode), then O^T += V^T P^T
  auto softmax_pv = [&](int step, const f32x4 (&s)[2][RT]) {
    const uint8_t* kl = smem + (step % NS) * STAGE;
    const uint8_t* vl = kl + KT * D;
    const float* ksl = (const float*)(kl + 2 * KT * D);
    const float* vsl = ksl + KT;
    const int kb0 = k_begin + step * KT;
    // V^T operands: transposed reads issued first, used after the softmax
    i32x2 vw[NT];
    {
      const uint8_t* rp = vl + tr_row * D + (r16 & 1) * 8;
#pragma unroll
      for (int t = 0; t < NT; ++t) vw[t] = lds_read_tr8(rp + ((t ^ tr_swz) << 4));
    }
    // per-token-head scales of the lane's 8 keys (4kg + r of each 16-key tile), one vector read each
    float ks[8], vs[8];
    if constexpr (PTH) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const float4 k4 = *(const float4*)(ksl + kt * 16 + 4 * kg);
        const float4 v4 = *(const float4*)(vsl + kt * 16 + 4 * kg);
        ks[4 * kt] = k4.x; ks[4 * kt + 1] = k4.y; ks[4 * kt + 2] = k4.z; ks[4 * kt + 3] = k4.w;
        vs[4 * kt] = v4.x; vs[4 * kt + 1] = v4.y; vs[4 * kt + 2] = v4.z; vs[4 * kt + 3] = v4.w;
      }
    }
    const bool full = wave_rows_full && kb0 >= vis_lo && kb0 + KT <= vis_hi && kb0 + KT <= it.L;
    bf16x8 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kt = e >> 2, r = e & 3;
        float v = s[kt][rt][r] * xscale;
        if constexpr (PTH) v *= ks[e];
        if constexpr (CAP) v = a.softcap * kLog2e * tanh_via_exp2(v * a.inv_softcap);
        x[e] = v;
      }
      if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = kb0 + (e >> 2) * 16 + 4 * kg + (e & 3);
          if (!(j >= lo_r[rt] && j < hi_r[rt])) x[e] = -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = max_over_rows(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m[rt] + 8.0f) != 0) {
        const float m_new = fmaxf(m[rt], mx);
        const float alpha = fast_exp2(m[rt] - (m_new == -INFINITY ? 0.0f : m_new));
        l[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] *= alpha;
        m[rt] = m_new;
      }
      const float m_use = m[rt] == -INFINITY ? 0.0f : m[rt];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pe = fast_exp2(x[e] - m_use);
        psum += pe;
        // a masked key may have an unwritten scale slot: select, do not multiply, its zero
        if constexpr (PTH) pe = x[e] == -INFINITY ? 0.0f : pe * vs[e];
        pb[rt][e] = (__bf16)pe;
      }
      l[rt] += psum;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 va = widen8<DT>((uint32_t)vw[t].x, (uint32_t)vw[t].y);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][t] = mfma16x16x32(va, pb[rt], acc[rt][t]);
    }
  };

  // ---- software pipeline: step t's softmax and PV product run while the QK^T product of step
  // t + 1 is in the matrix cores. Stages t and t + 1 are read during iteration t; the copies of
  // stages t + 2 .. t + NS - 1 are in flight.
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < n_steps) issue(s0);
  f32x4 s_cur[2][RT];
  if (n_steps > 0) {
    wait_vmcnt(min(NS - 2, n_steps - 1) * ipw_me);
    __syncthreads();  // stage 0 landed for every wave
    qk(0, s_cur);
  }
  for (int step = 0; step < n_steps; ++step) {
    f32x4 s_next[2][RT];
    if (step + 1 < n_steps) {
      // stage step + 1 is done once only the copies of later stages are outstanding
      const int issued = min(n_steps, step + NS - 1);
      wait_vmcnt((issued - step - 2) * ipw_me);
      __syncthreads();  // every wave's copies of stage step + 1 landed; every wave left step - 1
      if (step + NS - 1 < n_steps) issue(step + NS - 1);  // into the stage step - 1 used
      qk(step + 1, s_next);
    }
    softmax_pv(step, s_cur);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s_cur[kt][rt] = s_next[kt][rt];
  }

  // ---- normalise and write the rows
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = sum_over_rows(l[rt]);
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
  if (a.softcap > 0.0f)
    hipLaunchKernelGGL((prefill_kernel<D, DT, MODE, true>), dim3(h.num_pf_items), dim3(pf_waves(D) * 64), h.pf_lds_bytes, st, p);
  else
    hipLaunchKernelGGL((prefill_kernel<D, DT, MODE, false>), dim3(h.num_pf_items), dim3(pf_waves(D) * 64), h.pf_lds_bytes, st, p);
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
