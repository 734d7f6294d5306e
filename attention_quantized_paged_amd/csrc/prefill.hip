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
  float* scratch;     // partial results of split items: O of slot s at s * D, (m, l) at num_slots * D + 2 s
  int64_t num_slots;
  int64_t page_bytes, block_bytes;
  int32_t block_size, num_kv_heads, num_q_heads, group, max_blocks, num_blocks;
  int32_t window;
  float logit_scale;  // sm_scale * k_scale (per tensor) or sm_scale (per token-head)
  float softcap, inv_softcap;
  float v_scale;
  const float* alibi;  // [num_q_heads] slopes or null
  const float* sinks;  // [num_q_heads] sink logits or null
  uint32_t bs_magic;   // key / block_size = div_invariant(key, bs_magic, bs_shift) (block_size >= 2)
  int32_t bs_shift;
  float inv_bs;        // 1 / block_size (float): row quotients where tiles span blocks
};

// 16-byte chunk swizzle of a staged row: chunk c of row `row` is stored at chunk
// c ^ swz(row). Rows are ROWB bytes; 256 bytes span all LDS banks, so rows that share banks
// (same row / (256 / ROWB) residue) get different chunk offsets, and the second 16-key tile gets
// the upper half of the offsets. This keeps the K-operand reads (16 rows, one chunk) and the
// transposed V reads (8 rows of two tiles, one chunk) free of bank conflicts.
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  constexpr int CPR = ROWB / 16;                        // chunks per row
  constexpr int RPL = ROWB >= 256 ? 1 : 256 / ROWB;     // rows per 256 bytes
  return ((row / RPL) % CPR) ^ (((row >> 4) & 1) * (CPR / 2));
}

// GBS: the block size is not a multiple of 16, so a 16-key tile may span several blocks (up to
// 16): its rows are copied from their own blocks, its scales likewise in 4-byte copies, and the
// absent rows of a tile are masked row by row.
template <int D, int DT, int MODE, bool CAP, int ROWS, bool GBS>
__global__ __launch_bounds__(pf_waves(D) * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2))) void prefill_kernel(PfArgs a) {
  constexpr int NT = D / 16;
  constexpr int QS = D / 32;
  constexpr int WAVES = pf_waves(D);
  constexpr int RT = ROWS / (16 * WAVES);         // 16-row MFMA column blocks per wave
  static_assert(RT >= 1 && ROWS % (16 * WAVES) == 0, "rows must split evenly over the waves");
  constexpr int RPW = 16 * RT;                    // query rows per wave
  constexpr int KT = kPfKvTile;                   // keys per step (two 16-key tiles)
  constexpr int EB = DT == AQP_KV_AUTO ? 2 : 1;   // bytes per stored element (bf16 when unquantised)
  constexpr int NS = pf_stages(D, EB);            // LDS ring stages
  constexpr int ROWB = D * EB;                    // bytes of one staged key row
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  constexpr int STAGE = 2 * KT * ROWB + pf_stage_scale_bytes(D, MODE, EB);  // K rows, V rows, K scales, V scales
  constexpr int KV_INSTR = KT * CPR / 64;         // 1 KB copies per K (or V) step
  constexpr int IPW = 2 * KV_INSTR / WAVES;       // K+V copies per wave per step
  static_assert(IPW >= 1 && (2 * KV_INSTR) % WAVES == 0, "copies must split evenly over the waves");
  // bf16 operand images: the MFMA A operands of one step, 64 lanes x 16 bytes per 1 KB block,
  // written once per work-group and read by every wave
  constexpr int IMG = KT * D * 2;                 // one K (or V) image of a step
  constexpr int KIMG = NS * STAGE;                // two K images after the ring
  constexpr int VSLOT = IMG + pf_vslot_scale_bytes(EB);  // V image + the step's K and V scales
  constexpr int VIMG = KIMG + 2 * IMG;            // two V slots
  constexpr int KBLK = 2 * QS;                    // K blocks per image: [key tile][depth slice]
  constexpr int KB_PW = KBLK / WAVES;             // K blocks each wave converts
  constexpr int VB_PW = NT / WAVES;               // V blocks each wave converts
  static_assert(KB_PW >= 1 && KBLK % WAVES == 0 && VB_PW >= 1 && NT % WAVES == 0, "blocks must split evenly");
  constexpr int PTH = MODE == AQP_SCALE_PER_TOKEN_HEAD ? 1 : 0;
  constexpr int PG = MODE == AQP_SCALE_PER_GROUP ? 1 : 0;
  constexpr int NG = D / AQP_SCALE_GROUP;          // scale groups of a row (per-group mode)
  constexpr int SCH = 64 * NG;                     // bytes of one 16-key tile's group scales
  // scale copies per step (64 x 4 bytes each where tiles span blocks)
  constexpr int SCI = PTH ? 1 : (PG ? (GBS ? NG : (4 * SCH + 1023) / 1024) : 0);
  static_assert(EB == 1 || (!PTH && !PG), "the unquantised cache has no scales");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const PfItem it = load_const(as_const(a.items) + blockIdx.x);
  if (it.q_hi <= it.q_lo) return;  // an empty item (launch-order padding)
  const int G = a.group;
  const int nh = it.nheads;  // q heads per token in this item
  const int ntok = it.q_hi - it.q_lo;
  const cptr<int32_t> bt = as_const(a.block_tables) + (int64_t)it.seq * a.max_blocks;
  const uint8_t* kbase = a.cache + (int64_t)it.kvh * a.page_bytes;
  const uint8_t* vbase = a.cache + (int64_t)(a.num_kv_heads + it.kvh) * a.page_bytes;
  const uint32_t lds0 = lds_addr(smem);
  // copies this wave issues per step: its share of K/V, plus the scale copy on the last wave
  const int ipw_me = IPW + (wave == WAVES - 1 ? SCI : 0);

  // ---- rows of this lane (as MFMA column r16 of the wave's row tiles)
  int lo_r[RT], hi_r[RT];
  bool row_ok[RT];
  int64_t orow[RT];
  int pos_r[RT];      // position of the row's query
  float slope_r[RT];  // ALiBi slope of the row's head, in the log2 domain (0 without ALiBi)
  float sink_r[RT];   // sink logit of the row's head, in the log2 domain (-inf without sinks)
  bf16x8 qb[RT][QS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = wave * RPW + rt * 16 + r16;
    const int tl = row / nh, g = it.head0 + row - (row / nh) * nh;
    row_ok[rt] = tl < ntok;
    const int t = it.q_lo + (row_ok[rt] ? tl : 0);
    const int p = it.L - it.ql + t;
    hi_r[rt] = it.causal ? p + 1 : it.L;
    pos_r[rt] = p;
    const int hq = it.kvh * G + g;
    slope_r[rt] = a.alibi ? a.alibi[hq] * kLog2e : 0.0f;
    sink_r[rt] = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
    lo_r[rt] = (a.window > 0 && p - a.window + 1 > 0) ? p - a.window + 1 : 0;
    // a run of a split item sees only its own keys
    lo_r[rt] = max(lo_r[rt], it.split_lo);
    hi_r[rt] = min(hi_r[rt], it.split_hi);
    if (!row_ok[rt]) { lo_r[rt] = 0; hi_r[rt] = 0; }
    orow[rt] = ((int64_t)(it.q_start + t) * a.num_q_heads + it.kvh * G + g) * D;
    // (per group: depth 32*st + 8*kg + 0..7, so that MFMA step st covers scale group st)
    const uint16_t* qp = a.q + orow[rt] + (PG ? kg * 8 : kg * (D / 4));
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      uint4 u = *(const uint4*)(qp + st * (PG ? 32 : 8));
      if (!row_ok[rt]) u = make_uint4(0, 0, 0, 0);
      qb[rt][st] = __builtin_bit_cast(bf16x8, u);
    }
  }
  // the wave's rows cover tokens [tw0, tw1]: keys in [vis_lo, vis_hi) are visible to all of them
  const int tw0 = min(ntok - 1, (wave * RPW) / nh);
  const int tw1 = min(ntok - 1, (wave * RPW + RPW - 1) / nh);
  const bool wave_rows_full = (wave * RPW + RPW - 1) / nh < ntok;
  const int pw0 = it.L - it.ql + it.q_lo + tw0, pw1 = it.L - it.ql + it.q_lo + tw1;
  const int vis_hi = min(it.causal ? pw0 + 1 : it.L, it.split_hi);
  const int vis_lo = max((a.window > 0 && pw1 - a.window + 1 > 0) ? pw1 - a.window + 1 : 0, it.split_lo);
  // ---- key range of the whole item: first token's window start .. last token's end
  const int p_first = it.L - it.ql + it.q_lo;
  const int k_first = (a.window > 0 && p_first - a.window + 1 > 0) ? p_first - a.window + 1 : 0;
  const int k_begin = max((k_first / kTileKeys) * kTileKeys, it.split_lo);  // (split_lo: a step boundary)
  const int k_end = min(it.k_hi_max, it.split_hi);
  const int n_steps = (k_end - k_begin + KT - 1) / KT;
  const float xscale = CAP ? a.logit_scale : a.logit_scale * kLog2e;
  const int last_tile = ((it.L - 1) / kTileKeys) * kTileKeys;  // first key of the tile holding key L-1
  // block of key k (block_size 1, possible only with GBS, is outside the invariant-division method)
  auto key_block = [&](int k) {
    if constexpr (GBS) return a.block_size == 1 ? k : (int)div_invariant((uint32_t)k, a.bs_magic, a.bs_shift);
    else return (int)div_invariant((uint32_t)k, a.bs_magic, a.bs_shift);
  };
  // GBS: entries of the 16 blocks from the one holding key k0 (scalar loads, clamped to the
  // sequence's table row) and k0's row in its block; with block_size >= 16 a tile spans at most
  // two blocks, so two entries do
  struct Ents { i32x16 e; int r0; };
  auto tile_ents = [&](int k0) {
    Ents t;
    const int bi = key_block(k0);
    t.r0 = k0 - bi * a.block_size;
    if (a.block_size >= kTileKeys) {
      t.e[0] = bt[bi];
      t.e[1] = bt[min(bi + 1, a.max_blocks - 1)];
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) t.e[j] = bt[min(bi + j, a.max_blocks - 1)];
    }
    return t;
  };
  // GBS: block-table entry (as stored) and row of row n - r0 of a tile whose first key sits at
  // row r0 of its block (n = r0 + tile row: j = n / bs < 16 blocks on; 0 or 1 when block_size >= 16)
  auto row_entry = [&](const Ents& t, int n, int& rr) {
    int j;
    int32_t e;
    if (a.block_size >= kTileKeys) {
      j = n >= a.block_size ? 1 : 0;
      e = j ? t.e[1] : t.e[0];
    } else {
      j = small_quot(n, a.inv_bs);
      e = sel16(t.e, j);
    }
    rr = n - j * a.block_size;
    return e;
  };
  // ... and the block to read (block 0 for an entry outside the pool)
  auto row_block = [&](const Ents& t, int n, int& rr) {
    const int32_t e = row_entry(t, n, rr);
    return (uint32_t)e < (uint32_t)a.num_blocks ? e : 0;
  };
  // GBS: row masks of the issued steps, 32 bits per step (16 per tile) in slot step & 3, written
  // when the step's copies are issued (every wave issues every step)
  uint64_t ok_lo = 0, ok_hi = 0;
  // rows of tile tt (0, 1) of step s whose block-table entries name blocks of the pool (bit t: the
  // row copied for key k0 + t, i.e. key min(k0 + t, L - 1); keys of a block whose entry lies
  // outside it are absent: masked like keys out of range, and their codes, read from block 0
  // instead, never reach a product)
  using RowMask = std::conditional_t<GBS, uint32_t, bool>;  // without GBS a tile is whole or absent
  auto tile_rows = [&](int s, int tt) -> RowMask {
    if constexpr (GBS) {
      const uint64_t w = (s & 2) ? ok_hi : ok_lo;
      return (uint32_t)(w >> (32 * (s & 1) + 16 * tt)) & 0xFFFFu;
    } else {
      return (uint32_t)bt[key_block(min(k_begin + s * KT + kTileKeys * tt, last_tile))] < (uint32_t)a.num_blocks;
    }
  };

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
    // the step's two tiles, clamped to the tile of key L-1 (kb0 itself lies at or before it)
    const int t0 = min(kb0, last_tile), t1 = min(kb0 + kTileKeys, last_tile);
    Ents e0, e1;  // GBS: their block-table entries, read once for all of the step's copies
    if constexpr (GBS) {
      e0 = tile_ents(t0);
      e1 = tile_ents(t1);
      // the step's row masks: row t of tile tt holds key min(kb0 + 16 tt + t, L - 1)
      uint32_t m2 = 0;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const Ents& en = tt ? e1 : e0;
        const int key = min(kb0 + kTileKeys * tt + (lane & 15), it.L - 1);  // in [t_tt, t_tt + 16)
        int rr;
        const int32_t e = row_entry(en, en.r0 + (key - (tt ? t1 : t0)), rr);
        const bool ok = (uint32_t)e < (uint32_t)a.num_blocks;
        m2 |= ((uint32_t)__builtin_amdgcn_ballot_w64(ok && lane < 16) & 0xFFFFu) << (16 * tt);
      }
      const int sh = 32 * (step & 1);
      if (step & 2) ok_hi = (ok_hi & ~(0xFFFFFFFFull << sh)) | ((uint64_t)m2 << sh);
      else ok_lo = (ok_lo & ~(0xFFFFFFFFull << sh)) | ((uint64_t)m2 << sh);
    }
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int ii = wave + WAVES * j;
      const int kv = ii / KV_INSTR;
      const int q0 = 64 * (ii % KV_INSTR);
      const int q = q0 + lane;
      const int row = q / CPR;
      const int lc = (q % CPR) ^ swz<ROWB>(row);
      // tile of this copy (uniform), clamped to the tile of key L-1
      const int tile_k0 = min(kb0 + ((q0 / CPR) & ~15), last_tile);
      const int key = min(kb0 + row, it.L - 1);  // in [tile_k0, tile_k0 + 16)
      const uint8_t* src;
      if constexpr (GBS) {
        const Ents& en = ((q0 / CPR) & 16) ? e1 : e0;  // (tile_k0 is t0 or t1 alike)
        int rr;
        const int32_t blk = row_block(en, en.r0 + (key - tile_k0), rr);
        src = (kv ? vbase : kbase) + (int64_t)blk * a.block_bytes + (int64_t)rr * ROWB + lc * 16;
      } else {
        const int tbi = key_block(tile_k0);
        const int tr0 = tile_k0 - tbi * a.block_size;
        int32_t blk = bt[tbi];
        if ((uint32_t)blk >= (uint32_t)a.num_blocks) blk = 0;  // invalid table entry: stay in the pool
        src = (kv ? vbase : kbase) + (int64_t)blk * a.block_bytes + (int64_t)(tr0 + (key - tile_k0)) * ROWB + lc * 16;
      }
      dma16_to_lds(src, sbase + (uint32_t)(kv * KT * ROWB + q0 * 16));
    }
    if constexpr (GBS && (PTH || PG)) {
      if (wave == WAVES - 1) {
        // row by row, 4 bytes per lane: per token-head [K scales of the 32 keys][V scales]; per
        // group [K tile 0][K tile 1][V tile 0][V tile 1], 16 rows x NG floats each
#pragma unroll
        for (int c = 0; c < SCI; ++c) {
          const int idx = 64 * c + lane;
          const int per = 16 * (PTH ? 1 : NG);           // floats of one (tile, K or V)
          const int c2 = idx / per, rem = idx - c2 * per;
          const int tl = c2 & 1, kv = c2 >> 1;
          const int row = PTH ? rem : rem / NG, g = PTH ? 0 : rem % NG;
          const int tk0 = tl ? t1 : t0;
          const int key = min(kb0 + 16 * tl + row, it.L - 1);  // in [tk0, tk0 + 16)
          int rr0, rr1;
          const int32_t b0 = row_block(e0, e0.r0 + (key - tk0), rr0);
          const int32_t b1 = row_block(e1, e1.r0 + (key - tk0), rr1);
          const int32_t blk = tl ? b1 : b0;
          const int rr = tl ? rr1 : rr0;
          const uint8_t* src = (kv ? vbase : kbase) + (int64_t)blk * a.block_bytes + (int64_t)a.block_size * D +
                               4 * ((int64_t)rr * (PTH ? 1 : NG) + g);
          dma4_to_lds(src, sbase + (uint32_t)(2 * KT * ROWB + 256 * c));
        }
      }
    }
    if constexpr (PTH && !GBS) {
      if (wave == WAVES - 1) {
        // 16 lanes x 16 bytes: [K scales of the 32 keys][V scales], 4 scales per lane
        const int tl = (lane >> 2) & 1, part = lane & 3, kv = lane >> 3;
        const int t0 = min(kb0, last_tile), t1 = min(kb0 + 16, last_tile);
        const int bi0 = key_block(t0), bi1 = key_block(t1);
        int32_t b0 = bt[bi0], b1 = bt[bi1];
        if ((uint32_t)b0 >= (uint32_t)a.num_blocks) b0 = 0;
        if ((uint32_t)b1 >= (uint32_t)a.num_blocks) b1 = 0;
        const int tk0 = tl ? t1 : t0;
        const int32_t blk = tl ? b1 : b0;
        const int r0 = tk0 - (tl ? bi1 : bi0) * a.block_size;
        const uint8_t* src = (kv ? vbase : kbase) + (int64_t)blk * a.block_bytes + (int64_t)a.block_size * D +
                             4 * (r0 + 4 * part);
        if (lane < 16) dma16_to_lds(src, sbase + (uint32_t)(2 * KT * ROWB));
      }
    }
    if constexpr (PG && !GBS) {
      if (wave == WAVES - 1) {
        // [K scales of key tile 0][K tile 1][V tile 0][V tile 1]: 16 rows x NG floats each
        const int t0 = min(kb0, last_tile), t1 = min(kb0 + 16, last_tile);
        const int bi0 = key_block(t0), bi1 = key_block(t1);
        int32_t b0 = bt[bi0], b1 = bt[bi1];
        if ((uint32_t)b0 >= (uint32_t)a.num_blocks) b0 = 0;
        if ((uint32_t)b1 >= (uint32_t)a.num_blocks) b1 = 0;
#pragma unroll
        for (int j = 0; j < SCI; ++j) {
          const int o = 1024 * j + 16 * lane;
          const int c = o / SCH, w = o - (o / SCH) * SCH;
          const int tl = c & 1, kv = (c >> 1) & 1;
          const int r0 = (tl ? t1 : t0) - (tl ? bi1 : bi0) * a.block_size;
          const uint8_t* src = (kv ? vbase : kbase) + (int64_t)(tl ? b1 : b0) * a.block_bytes +
                               (int64_t)a.block_size * D + 4 * (int64_t)r0 * NG + w;
          if (o < 4 * SCH) dma16_to_lds(src, sbase + (uint32_t)(2 * KT * ROWB + 1024 * j));
        }
      }
    }
  };

  // transposed V read: row i of lane group kg is key (i < 4 ? 4kg + i : 16 + 4kg + i - 4)
  const int tr_i = r16 >> 1;
  const int tr_row = (tr_i < 4) ? (4 * kg + tr_i) : (16 + 4 * kg + tr_i - 4);
  const int tr_swz = swz<ROWB>(tr_row);

  // ---- widen the K codes of one step into its K image: block kt * QS + st holds, for lane l,
  // the 8 depth values kg * D/4 + 8 st .. +7 of key kt * 16 + l % 16 (the A operand of S^T = K Q^T)
  auto convert_k = [&](int step) {
    const uint8_t* kl = smem + (step % NS) * STAGE;
    uint8_t* img = smem + KIMG + (step & 1) * IMG + lane * 16;
#pragma unroll
    for (int j = 0; j < KB_PW; ++j) {
      const int blk = wave * KB_PW + j;
      const int kt = blk / QS, st = blk - (blk / QS) * QS;
      const int krow = kt * 16 + r16;
      const int dbyte = (kg * (D / 4) + st * 8) * EB;
      if constexpr (PG) {
        // per group: depth 32*st + 8*kg + 0..7 (group st), exact codes; the key's group scale
        // multiplies the product in the QK step
        const int gbyte = 32 * st + 8 * kg;
        const uint2 c = *(const uint2*)(kl + krow * ROWB + ((((gbyte >> 4) ^ swz<ROWB>(krow)) << 4) | (gbyte & 8)));
        *(bf16x8*)(img + blk * 1024) = widen8<DT>(c.x, c.y);
      } else if constexpr (EB == 1) {
        const uint2 c = *(const uint2*)(kl + krow * ROWB + ((((dbyte >> 4) ^ swz<ROWB>(krow)) << 4) | (dbyte & 8)));
        *(bf16x8*)(img + blk * 1024) = widen8<DT>(c.x, c.y);
      } else {
        // bf16 rows: the 16 bytes are the operand already
        *(uint4*)(img + blk * 1024) = *(const uint4*)(kl + krow * ROWB + (((dbyte >> 4) ^ swz<ROWB>(krow)) << 4));
      }
    }
  };
  // ---- widen the V codes of one step into its V image: block t holds, for lane l, dim
  // t * 16 + l % 16 of the 8 keys of lane group kg (the A operand of O^T += V^T P^T); the step's
  // K and V scales are copied next to it, so they outlive the ring stage
  // (ok0, ok1: bit t set when row t of the step's first (second) 16-key tile lies in a block of
  // the pool; the codes of an absent row become zeros)
  auto convert_v = [&](int step, RowMask ok0, RowMask ok1) {
    const uint8_t* kl = smem + (step % NS) * STAGE;
    uint8_t* slot = smem + VIMG + (step & 1) * VSLOT;
    // the lane's rows i < 4 are keys 4kg + i of the first tile, rows i >= 4 keys 4kg + i - 4 of
    // the second: one byte per row (codes), or a whole mask per row (16-bit elements)
    const uint32_t b0 = ((uint32_t)ok0 >> (4 * kg)) & 0xFu, b1 = ((uint32_t)ok1 >> (4 * kg)) & 0xFu;
    auto bytes = [](uint32_t b) {
      return ((b & 1u) ? 0xFFu : 0u) | ((b & 2u) ? 0xFF00u : 0u) | ((b & 4u) ? 0xFF0000u : 0u) | ((b & 8u) ? 0xFF000000u : 0u);
    };
    const uint32_t msk0 = GBS ? bytes(b0) : (ok0 ? 0xFFFFFFFFu : 0u), msk1 = GBS ? bytes(b1) : (ok1 ? 0xFFFFFFFFu : 0u);
    // row i of the lane present in its block (without GBS a tile's rows share one block)
    auto present_row = [&](int i) { return GBS ? (((i < 4 ? b0 : b1) >> (i & 3)) & 1) != 0 : (bool)(i < 4 ? ok0 : ok1); };
    if constexpr (EB == 1) {
      const uint8_t* rp = kl + KT * ROWB + tr_row * ROWB + (r16 & 1) * 8;
#pragma unroll
      for (int j = 0; j < VB_PW; ++j) {
        const int t = wave * VB_PW + j;
        i32x2 c = lds_read_tr8(rp + ((t ^ tr_swz) << 4));
        c.x &= (int)msk0;  // rows i < 4: keys of the first tile
        c.y &= (int)msk1;
        if constexpr (PG) {
          // element i is key row (i < 4 ? 4kg + i : 16 + 4kg + i - 4) at a head-dim column of
          // group t / 2: bf16(code * that key's scale); keys past L get 0
          const float* vsc = (const float*)(kl + 2 * KT * ROWB) + 2 * 16 * NG;
          const bf16x8 e = widen8<DT>((uint32_t)c.x, (uint32_t)c.y);
          bf16x8 r;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = i < 4 ? 4 * kg + i : 16 + 4 * kg + i - 4;
            const bool present = k_begin + step * KT + row < it.L && present_row(i);
            const float sc = present ? vsc[row * NG + (t >> 1)] : 0.0f;
            r[i] = (__bf16)((float)e[i] * sc);
          }
          *(bf16x8*)(slot + t * 1024 + lane * 16) = r;
        } else {
          *(bf16x8*)(slot + t * 1024 + lane * 16) = widen8<DT>((uint32_t)c.x, (uint32_t)c.y);
        }
      }
    } else {
      // bf16 rows: the lane's 8 keys of head-dim column t * 16 + r16, one 16-bit read each
      const uint8_t* vl = kl + KT * ROWB + (r16 & 7) * 2;
#pragma unroll
      for (int j = 0; j < VB_PW; ++j) {
        const int t = wave * VB_PW + j;
        uint32_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = i < 4 ? 4 * kg + i : 16 + 4 * kg + i - 4;
          e[i] = *(const uint16_t*)(vl + row * ROWB + (((2 * t + (r16 >> 3)) ^ swz<ROWB>(row)) << 4)) &
                 (GBS ? (present_row(i) ? 0xFFFFu : 0u) : (i < 4 ? msk0 : msk1));
        }
        *(uint4*)(slot + t * 1024 + lane * 16) =
            make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
      }
    }
    if constexpr (PTH) {
      if (wave == WAVES - 1 && lane < 16) *(uint4*)(slot + IMG + lane * 16) = *(const uint4*)(kl + 2 * KT * ROWB + lane * 16);
    }
  };

  // ---- the same two widenings (one-byte codes, per-tensor or per-token-head scales) in two
  // phases: every code read of both issued before any image write, so that the reads wait on one
  // LDS round trip together (an image write cannot be moved above a later ring read it might
  // alias, so the one-block-at-a-time form waits once per block)
  auto kv_codes = [&](int kstep, int vstep, uint2 (&kc)[KB_PW], i32x2 (&vc)[VB_PW]) {
    const uint8_t* kl = smem + (kstep % NS) * STAGE;
#pragma unroll
    for (int j = 0; j < KB_PW; ++j) {
      const int blk = wave * KB_PW + j;
      const int kt = blk / QS, st = blk - (blk / QS) * QS;
      const int krow = kt * 16 + r16;
      const int dbyte = kg * (D / 4) + st * 8;
      kc[j] = *(const uint2*)(kl + krow * ROWB + ((((dbyte >> 4) ^ swz<ROWB>(krow)) << 4) | (dbyte & 8)));
    }
    const uint8_t* rp = smem + (vstep % NS) * STAGE + KT * ROWB + tr_row * ROWB + (r16 & 1) * 8;
#pragma unroll
    for (int j = 0; j < VB_PW; ++j) vc[j] = lds_read_tr8(rp + (((wave * VB_PW + j) ^ tr_swz) << 4));
  };
  auto kv_images = [&](int kstep, int vstep, RowMask ok0, RowMask ok1, const uint2 (&kc)[KB_PW], const i32x2 (&vc)[VB_PW]) {
    uint8_t* img = smem + KIMG + (kstep & 1) * IMG + lane * 16;
#pragma unroll
    for (int j = 0; j < KB_PW; ++j) *(bf16x8*)(img + (wave * KB_PW + j) * 1024) = widen8<DT>(kc[j].x, kc[j].y);
    uint8_t* slot = smem + VIMG + (vstep & 1) * VSLOT;
    const uint32_t b0 = ((uint32_t)ok0 >> (4 * kg)) & 0xFu, b1 = ((uint32_t)ok1 >> (4 * kg)) & 0xFu;
    auto bytes = [](uint32_t b) {
      return ((b & 1u) ? 0xFFu : 0u) | ((b & 2u) ? 0xFF00u : 0u) | ((b & 4u) ? 0xFF0000u : 0u) | ((b & 8u) ? 0xFF000000u : 0u);
    };
    const uint32_t msk0 = GBS ? bytes(b0) : (ok0 ? 0xFFFFFFFFu : 0u), msk1 = GBS ? bytes(b1) : (ok1 ? 0xFFFFFFFFu : 0u);
#pragma unroll
    for (int j = 0; j < VB_PW; ++j)
      *(bf16x8*)(slot + (wave * VB_PW + j) * 1024 + lane * 16) = widen8<DT>((uint32_t)vc[j].x & msk0, (uint32_t)vc[j].y & msk1);
    if constexpr (PTH) {
      const uint8_t* kl = smem + (vstep % NS) * STAGE;
      if (wave == WAVES - 1 && lane < 16) *(uint4*)(slot + IMG + lane * 16) = *(const uint4*)(kl + 2 * KT * ROWB + lane * 16);
    }
  };

  // ---- K operands of one step from its K image: [key tile][depth slice]
  auto read_k = [&](int step, bf16x8 (&kw)[2][QS]) {
    const uint8_t* img = smem + KIMG + (step & 1) * IMG + lane * 16;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int st = 0; st < QS; ++st) kw[kt][st] = *(const bf16x8*)(img + (kt * QS + st) * 1024);
  };
  // ---- half h of the depth slices of S^T = K Q^T: [key tile kt][row tile rt]
  // (per group: `sstep` is the step S belongs to; each depth slice is group st, its product
  // scaled per key by the key's group scale from that step's ring stage, keys past L by 0)
  auto qk_half = [&](int h, const bf16x8 (&kw)[2][QS], f32x4 (&s)[2][RT], int sstep) {
    if constexpr (PG) {
      const float* ksc = (const float*)(smem + (sstep % NS) * STAGE + 2 * KT * ROWB);
      const int kb = k_begin + sstep * KT;
#pragma unroll
      for (int st = h * (QS / 2); st < (h + 1) * (QS / 2); ++st)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          float sc[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kt * 16 + 4 * kg + r;
            sc[r] = kb + key < it.L ? ksc[key * NG + st] : 0.0f;
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const f32x4 sg = mfma16x16x32(kw[kt][st], qb[rt][st], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) s[kt][rt][r] = (st == 0 ? 0.0f : s[kt][rt][r]) + sc[r] * sg[r];
          }
        }
    } else {
#pragma unroll
      for (int st = h * (QS / 2); st < (h + 1) * (QS / 2); ++st)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            s[kt][rt] = mfma16x16x32(kw[kt][st], qb[rt][st], st == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kt][rt]);
    }
  };

  // ---- prologue: stages 0 and 1 widened, S of step 0
  // (the software pipeline below: iteration t, after one barrier, puts the copies of step t + NS
  // into the ring stage step t left (half the waves at once, the other half mid-step), computes
  // S of step t + 1 in the matrix cores while the softmax of step t runs, then the PV product of
  // step t while K of step t + 2 and V of step t + 1 are widened into their images. Each image is
  // written one iteration before it is read, so one barrier per step orders both. The last
  // iteration computes an S it does not use.)
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0)
    if (s0 < n_steps) issue(s0);
  f32x4 s_cur[2][RT];
  if (n_steps > 0) {
    wait_vmcnt(max(0, min(NS, n_steps) - 2) * ipw_me);
    __syncthreads();  // stages 0 and 1 landed for every wave
    convert_k(0);
    convert_k(1);
    convert_v(0, tile_rows(0, 0), tile_rows(0, 1));
    __syncthreads();
    bf16x8 kw[2][QS];
    read_k(0, kw);
    qk_half(0, kw, s_cur, 0);
    qk_half(1, kw, s_cur, 0);
  }
  RowMask cur_ok0 = n_steps > 0 ? tile_rows(0, 0) : RowMask(0), cur_ok1 = n_steps > 0 ? tile_rows(0, 1) : RowMask(0);
  for (int step = 0; step < n_steps; ++step) {
    // validity of the next step's tiles (its V codes are widened in this iteration; its keys are
    // masked in the next)
    const RowMask nxt_ok0 = tile_rows(step + 1, 0), nxt_ok1 = tile_rows(step + 1, 1);
    // stage step + 2 landed once only the copies of later stages are outstanding
    const int issued = min(n_steps, step + NS);
    // (issued - step - 3 is 1, or 0 at the last steps: compile-time counts, no runtime switch)
    if (issued - step - 3 <= 0) wait_vmcnt_c<0>();
    else if (SCI > 0 && wave == WAVES - 1) wait_vmcnt_c<IPW + SCI>();
    else wait_vmcnt_c<IPW>();
    __syncthreads();  // every wave's copies of stage step + 2 landed; every wave left iteration step - 1
    // the copies of step + NS go into the stage of step, whose codes are widened: even waves issue
    // theirs here, odd waves before the PV product, so the memory pipeline takes them in two
    // bursts and fewer waves stall on a full request queue at once
    if ((wave & 1) == 0 && step + NS < n_steps) issue(step + NS);
    bf16x8 kw[2][QS];
    read_k(step + 1, kw);

    const uint8_t* slot = smem + VIMG + (step & 1) * VSLOT;
    const int kb0 = k_begin + step * KT;
    // logits of step (log2 domain), masked where a step is not visible to all of the wave's rows
    float ks[8], vs[8];
    if constexpr (PTH) {
      const float* ksl = (const float*)(slot + IMG);
      const float* vsl = ksl + KT;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const float4 k4 = *(const float4*)(ksl + kt * 16 + 4 * kg);
        const float4 v4 = *(const float4*)(vsl + kt * 16 + 4 * kg);
        ks[4 * kt] = k4.x; ks[4 * kt + 1] = k4.y; ks[4 * kt + 2] = k4.z; ks[4 * kt + 3] = k4.w;
        vs[4 * kt] = v4.x; vs[4 * kt + 1] = v4.y; vs[4 * kt + 2] = v4.z; vs[4 * kt + 3] = v4.w;
      }
    }
    float x[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = s_cur[e >> 2][rt][e & 3] * xscale;
        if constexpr (PTH) v *= ks[e];
        if constexpr (CAP) v = a.softcap * kLog2e * tanh_via_exp2(v * a.inv_softcap);
        x[rt][e] = v;
      }
    if (a.alibi) {
      // + slope * (key - position), after the soft-cap
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int base = kb0 + 4 * kg - pos_r[rt];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[rt][e] += slope_r[rt] * (float)(base + (e >> 2) * 16 + (e & 3));
      }
    }
    const bool full = wave_rows_full && kb0 >= vis_lo && kb0 + KT <= vis_hi && kb0 + KT <= it.L &&
                      (GBS ? ((uint32_t)cur_ok0 & (uint32_t)cur_ok1) == 0xFFFFu : (cur_ok0 && cur_ok1));
    if (!full) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = kb0 + (e >> 2) * 16 + 4 * kg + (e & 3);
          const RowMask okm = (e >> 2) == 0 ? cur_ok0 : cur_ok1;
          const bool present = GBS ? (((uint32_t)okm >> (4 * kg + (e & 3))) & 1) != 0 : (bool)okm;
          if (!(j >= lo_r[rt] && j < hi_r[rt] && present)) x[rt][e] = -INFINITY;
        }
    }

    // first half of S of step + 1 while the row maxima of step are taken
    f32x4 s_next[2][RT];
    qk_half(0, kw, s_next, step + 1);
    float mx[RT];
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float v = x[rt][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) v = fmaxf(v, x[rt][e]);
      mx[rt] = max_over_rows(v);
      grow = grow || (mx[rt] > m[rt] + 8.0f);
    }
#pragma unroll
    for (int i = 0; i < 2 * RT * (QS / 2); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    // lazy rescaling: the reference maximum moves only when a row's logits exceed it by 8
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float m_new = fmaxf(m[rt], mx[rt]);
        const float alpha = fast_exp2(m[rt] - (m_new == -INFINITY ? 0.0f : m_new));
        l[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] *= alpha;
        m[rt] = m_new;
      }
    }

    // second half of S of step + 1 while the probabilities of step are formed; the V operands
    // of step are read meanwhile
    const uint8_t* vimg = slot + lane * 16;
    bf16x8 vw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) vw[t] = *(const bf16x8*)(vimg + t * 1024);
    qk_half(1, kw, s_next, step + 1);
    bf16x8 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float m_use = m[rt] == -INFINITY ? 0.0f : m[rt];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pe = fast_exp2(x[rt][e] - m_use);
        psum += pe;
        // a masked key may have an unwritten scale slot: select, do not multiply, its zero
        if constexpr (PTH) pe = x[rt][e] == -INFINITY ? 0.0f : pe * vs[e];
        pb[rt][e] = (__bf16)pe;
      }
      l[rt] += psum;
    }

    if ((wave & 1) == 1 && step + NS < n_steps) issue(step + NS);
    // O^T += V^T P^T of step while K of step + 2 and V of step + 1 are widened
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][t] = mfma16x16x32(vw[t], pb[rt], acc[rt][t]);
    if constexpr (EB == 1 && !PG) {
      uint2 kc[KB_PW];
      i32x2 vc[VB_PW];
      kv_codes(step + 2, step + 1, kc, vc);
      kv_images(step + 2, step + 1, nxt_ok0, nxt_ok1, kc, vc);
    } else {
      convert_k(step + 2);
      convert_v(step + 1, nxt_ok0, nxt_ok1);
    }
    // issue order of this block: half the V reads, then each matrix op of S with four vector ops
    // of the softmax, then each PV matrix op with one LDS read and one vector op
    __builtin_amdgcn_sched_group_barrier(0x100, NT / 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * RT * (QS / 2); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
#pragma unroll
    for (int i = 0; i < NT * RT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }

#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s_cur[kt][rt] = s_next[kt][rt];
    cur_ok0 = nxt_ok0;
    cur_ok1 = nxt_ok1;
  }

  // ---- normalise and write the rows (a run of a split item: its partial results instead)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float lt = sum_over_rows(l[rt]);
    if (!row_ok[rt]) continue;
    if (it.slot >= 0) {
      const int64_t slot = (int64_t)it.slot + wave * RPW + rt * 16 + r16;
      float* pp = a.scratch + slot * D;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *(float4*)(pp + t * 16 + 4 * kg) = make_float4(acc[rt][t][0] * a.v_scale, acc[rt][t][1] * a.v_scale,
                                                       acc[rt][t][2] * a.v_scale, acc[rt][t][3] * a.v_scale);
      if (kg == 0) {
        float* ml = a.scratch + a.num_slots * D + slot * 2;
        ml[0] = m[rt];
        ml[1] = lt;
      }
      continue;
    }
    float f = 1.0f;
    if (a.sinks) {
      // the sink logit joins the normaliser: rescale to the larger of it and the row's reference
      const float M = fmaxf(m[rt], sink_r[rt]);
      f = fast_exp2(m[rt] - M);
      lt = lt * f + fast_exp2(sink_r[rt] - M);
    }
    // a row with no key left (every block of its range outside the pool) and no sink writes 0
    const float norm = lt > 0.0f ? a.v_scale * f / lt : 0.0f;
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
  p.scratch = a.scratch;
  p.num_slots = h.num_slots;
  p.page_bytes = a.page_bytes;
  p.block_bytes = a.block_bytes;
  p.block_size = a.block_size;
  invariant_divisor((uint32_t)a.block_size, &p.bs_magic, &p.bs_shift);
  p.inv_bs = 1.0f / (float)a.block_size;
  p.num_kv_heads = a.num_kv_heads;
  p.num_q_heads = a.num_q_heads;
  p.group = a.group;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = h.num_blocks;
  p.window = a.window;
  p.logit_scale = MODE == AQP_SCALE_PER_TENSOR ? a.sm_scale * a.k_scale : a.sm_scale;
  p.softcap = a.softcap;
  p.inv_softcap = a.softcap > 0.0f ? 1.0f / a.softcap : 0.0f;
  p.v_scale = MODE == AQP_SCALE_PER_TENSOR ? a.v_scale : 1.0f;
  p.alibi = a.alibi_slopes;
  p.sinks = a.sinks;
  const dim3 grid(h.num_pf_items), block(pf_waves(D) * 64);
  const bool gbs = a.block_size % kTileKeys != 0;  // tiles may span blocks
#define AQP_PF_GO(CAPV, ROWSV)                                                                                    \
  if (gbs)                                                                                                        \
    hipLaunchKernelGGL((prefill_kernel<D, DT, MODE, CAPV, ROWSV, true>), grid, block, h.pf_lds_bytes, st, p);  \
  else                                                                                                            \
    hipLaunchKernelGGL((prefill_kernel<D, DT, MODE, CAPV, ROWSV, false>), grid, block, h.pf_lds_bytes, st, p);
  if (h.pf_rows == kPfRows) {
    if (a.softcap > 0.0f) {
      AQP_PF_GO(true, kPfRows)
    } else {
      AQP_PF_GO(false, kPfRows)
    }
  } else if constexpr (pf_waves(D) * 16 <= kPfRowsSmall) {
    if (h.pf_rows != kPfRowsSmall) {
      set_error("aqp_paged_attention: schedule rows per prefill item %d not built", h.pf_rows);
      return AQP_ERR_SCHEDULE_MISMATCH;
    }
    if (a.softcap > 0.0f) {
      AQP_PF_GO(true, kPfRowsSmall)
    } else {
      AQP_PF_GO(false, kPfRowsSmall)
    }
  } else {
    set_error("aqp_paged_attention: schedule rows per prefill item %d not built at head_dim %d", h.pf_rows, D);
    return AQP_ERR_SCHEDULE_MISMATCH;
  }
#undef AQP_PF_GO
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
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_AUTO) return pf_d<AQP_KV_AUTO, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E4M3) return pf_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E5M2) return pf_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_INT8) return pf_d<AQP_KV_INT8, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E4M3) return pf_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_INT8) return pf_d<AQP_KV_INT8, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E5M2) return pf_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_INT8) return pf_d<AQP_KV_INT8, AQP_SCALE_PER_GROUP>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_FP8_E4M3) return pf_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_GROUP>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_FP8_E5M2) return pf_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_GROUP>(a, st);
  set_error("aqp_paged_attention: dtype %d with scale mode %d is not built", dtype, mode);
  return AQP_ERR_UNSUPPORTED;
}

}  // namespace aqp
