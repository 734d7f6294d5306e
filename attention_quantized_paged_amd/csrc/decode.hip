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
//  * a wave takes 16-key tiles w, w+4, ... of each of the work-group's segments, one
//    stream of tiles across segment boundaries;
//  * each tile's K and V codes (and per-token-head scales) are copied straight from HBM
//    into the wave's own LDS ring with global_load_lds (16-byte chunks, XOR-swizzled
//    per row so the operand reads below are free of bank conflicts), dec_stages(D) - 1
//    tiles ahead of the one being computed; the stream does not drain at segment ends,
//    so the copies of the next segment overlap the merge of the current one. The
//    segment's Q rows travel the same way, into a per-wave Q slot;
//  * K: each lane reads D/4 code bytes of one key, widens them to bf16 in registers and
//    feeds v_mfma_f32_16x16x32_bf16 as S^T = K * Q^T with the group's q heads as the
//    16 MFMA columns;
//  * scale folding: per tensor, k_scale goes into the logit scale and v_scale
//    into the final normalisation; per token-head, each key's scale multiplies
//    its logit and each value's scale its probability;
//  * softmax: running max / sum in the exp2 domain, reduced across the four lanes that
//    share a head with lane permutes; lazy rescaling; with a ring of three or more tiles, two of
//    the wave's tiles per loop iteration share one reduction and one rescale check (their S
//    products are independent);
//  * V: ds_read_b64_tr_b8 hands each lane 4 keys of one head-dim column for two column
//    tiles at once: the key-contiguous operand that O^T = V^T * P^T on
//    v_mfma_f32_16x16x16_bf16 needs, so the probabilities stay in the registers the
//    QK^T product left them in;
//  * the four waves' (m, l, O) are merged in LDS; the result is either the
//    output row (bf16) or a partial slot for the split-KV merge kernel.
#include "device_common.h"

namespace aqp {

struct DecArgs {
  const uint8_t* cache;
  const uint16_t* q;
  const int32_t* block_tables;
  const DecSeg* segs;
  const int32_t* wg_start;  // segments of work-group b: [wg_start[b], wg_start[b + 1])
  const DecSeg* first;      // first segment of work-group b (segs[wg_start[b]])
  float* scratch;
  uint16_t* out;
  int64_t page_bytes, block_bytes;
  int32_t block_size, num_kv_heads, num_q_heads, group, max_blocks, group_heads, num_blocks;
  float inv_bs;       // 1 / block_size (float): row quotients where tiles span blocks
  int64_t num_slots;  // partial-result slots of the scratch ((m, l) follow all slots' O)
  float logit_scale;  // sm_scale * k_scale (per tensor) or sm_scale (per token-head)
  float softcap, inv_softcap;
  float v_scale;      // per tensor; 1 per token-head
  const int32_t* seq_lens;  // keys of each sequence (schedule copy): the query sits at L - 1
  const float* alibi;       // [num_q_heads] slopes or null
  const float* sinks;       // [num_q_heads] sink logits or null
};

// Stored 16-byte chunk of logical chunk c in staged row `row` (rows of ROWB bytes): c ^ dec_swz(row).
// Rows that fall on the same LDS banks (same row / (256 / ROWB) residue) get distinct offsets, so
// the 16 rows of a K operand read and the 4 x 2 rows of a transposed V read hit distinct banks.
template <int ROWB>
__device__ __forceinline__ int dec_swz(int row) {
  constexpr int CPR = ROWB / 16;
  constexpr int RPB = ROWB >= 256 ? 1 : 256 / ROWB;
  return (row / RPB) % CPR;
}

// LDS barrier for the work-group that orders LDS traffic only (the global stores of the merge
// need no ordering against the other waves, and the copies in flight must not be waited for).
__device__ __forceinline__ void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Merge of the four compute waves' (O, m, l) of one segment, left in LDS as [wave][head][merge_stride(D)],
// into the output rows (bf16) or the segment's partial slot. Lane (r16, kg) handles head r16 and
// head-dim elements t * 16 + 4 kg + r, the layout the waves' accumulators have.
template <int D>
__device__ __forceinline__ void merge_store(const DecArgs& a, const float* mg, int gh, const DecSeg& sg, int r16, int kg) {
  constexpr int NT = D / 16;
  if (r16 >= sg.nheads) return;
  float mw[kDecWaves], lw[kDecWaves];
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const float* src = mg + (w * gh + r16) * merge_stride(D);
    mw[w] = src[D];
    lw[w] = src[D + 1];
  }
  float M = mw[0];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, mw[w]);
  const float M_use = M == -INFINITY ? 0.0f : M;
  float f[kDecWaves], L = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    f[w] = fast_exp2(mw[w] - M_use);
    L += f[w] * lw[w];
  }
  f32x4 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const f32x4 src = *(const f32x4*)(mg + (w * gh + r16) * merge_stride(D) + t * 16 + 4 * kg);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[t][r] += f[w] * src[r];
    }
  }
  const int hq = sg.kvh * a.group + sg.head0 + r16;
  if (sg.part < 0) {
    float fs = 1.0f;
    if (a.sinks) {
      // the sink logit joins the normaliser (log2 domain); M_use is the reference of o and L
      const float s2 = a.sinks[hq] * kLog2e;
      const float Mx = fmaxf(M_use, s2);
      fs = fast_exp2(M_use - Mx);
      L = L * fs + fast_exp2(s2 - Mx);
    }
    // a head with no key left (every block of its range outside the pool) and no sink writes 0
    const float norm = L > 0.0f ? a.v_scale * fs / L : 0.0f;
    uint16_t* op = a.out + ((int64_t)sg.q_tok * a.num_q_heads + hq) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16_rne(o[t][0] * norm) | ((uint32_t)f32_to_bf16_rne(o[t][1] * norm) << 16);
      w.y = (uint32_t)f32_to_bf16_rne(o[t][2] * norm) | ((uint32_t)f32_to_bf16_rne(o[t][3] * norm) << 16);
      *(uint2*)(op + t * 16 + 4 * kg) = w;
    }
  } else {
    // partial slot part * group_heads + head: O at [slot][D], (m, l) at [slot][2] after all O slots
    float* pp = a.scratch + ((int64_t)sg.part * a.group_heads + r16) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *(float4*)(pp + t * 16 + 4 * kg) = make_float4(o[t][0] * a.v_scale, o[t][1] * a.v_scale, o[t][2] * a.v_scale,
                                                     o[t][3] * a.v_scale);
    if (kg == 0) {
      float* ml = a.scratch + a.num_slots * D + ((int64_t)sg.part * a.group_heads + r16) * 2;
      ml[0] = M;
      ml[1] = L;
    }
  }
}

// GBS: the block size is not a multiple of 16, so a tile's 16 rows may lie in several blocks
// (up to 16): each row is copied from its own block, its scales likewise, and the absent rows
// of a tile are masked row by row.
template <int D, int DT, int MODE, bool CAP, bool GBS>
__global__ __launch_bounds__((kDecWaves + 1) * 64) __attribute__((amdgpu_waves_per_eu(dec_waves_per_simd(D)))) void decode_kernel(DecArgs a) {
  constexpr int NT = D / 16;   // 16-wide head-dim tiles of the output
  constexpr int QS = D / 32;   // 32-deep MFMA steps of QK^T
  constexpr int EB = DT == AQP_KV_AUTO ? 2 : 1;   // bytes per stored element (bf16 when unquantised)
  constexpr int ROWB = D * EB;                    // bytes of one staged key row
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per staged row
  constexpr int STEP = kDecWaves * kDecIterKeys;  // keys between a wave's consecutive tiles
  constexpr int PTH = MODE == AQP_SCALE_PER_TOKEN_HEAD ? 1 : 0;
  constexpr int PG = MODE == AQP_SCALE_PER_GROUP ? 1 : 0;
  constexpr int NG = D / AQP_SCALE_GROUP;          // scale groups of a row (per-group mode)
  constexpr int NS = dec_stages(D, EB);           // ring slots per wave
  constexpr int NQ = 1;                           // Q slots per wave
  constexpr int TB = kDecIterKeys * ROWB;         // bytes of one K (or V) tile
  constexpr int KI = TB / 1024;                   // 1 KB copies per K (or V) tile
  constexpr int SLOT = dec_slot_bytes(D, MODE, EB);  // K tile, V tile, K scales, V scales
  // copies per tile: K and V codes, then the scales (one 16-byte copy per tile; row by row in
  // 4-byte copies where tiles span blocks: 32 per token-head, 32 NG per group)
  constexpr int SCC = GBS ? (PTH ? 1 : (PG ? (NG + 1) / 2 : 0)) : PTH + PG;
  constexpr int IPT = 2 * KI + SCC;
  static_assert(KI >= 1 && IPT * (NS - 1) <= 63, "tile copies and waits");
  static_assert(EB == 1 || (!PTH && !PG), "the unquantised cache has no scales");
  static_assert(8 * NG <= 64, "one copy holds a tile's group scales");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int gh = a.group_heads;
  const int QB = gh * D * 2;  // bytes of a Q slot: the group's q rows, bf16
  uint8_t* ring = smem + wave * (NS * SLOT);
  uint8_t* qslots = smem + kDecWaves * NS * SLOT + wave * (NQ * QB);
  float* mg = (float*)(smem + kDecWaves * NS * SLOT + kDecWaves * NQ * QB);  // [wave][head][merge_stride(D)]
  const uint32_t ring_lds = lds_addr(ring), q_lds = lds_addr(qslots);
  const int s_begin = as_const(a.wg_start)[blockIdx.x], s_end = as_const(a.wg_start)[blockIdx.x + 1];
  const DecSeg first_sg = load_const(as_const(a.first) + blockIdx.x);

  if (wave == kDecWaves) {
    // ---- the merging wave: takes part in the two barriers of every segment, merges the compute
    // waves' (O, m, l) and writes the result while they go on with the next segment (so the
    // stores never hold up a wave that has copies in flight)
    for (int si = s_begin; si < s_end; ++si) {
      const DecSeg sg = load_const(as_const(a.segs) + si);
      block_sync_lds();
      block_sync_lds();
      merge_store<D>(a, mg, gh, sg, r16, kg);
    }
    return;
  }

  // transposed-read address of this lane: rows i = 0..3 and 4..7 are keys 4kg + (i & 3) at
  // logical chunks 2 t2 and 2 t2 + 1, so one read yields the operands of two head-dim tiles
  const int tr_i = r16 >> 1;
  const int tr_row = 4 * kg + (tr_i & 3);
  const int tr_hi = tr_i >> 2;
  const int tr_base = tr_row * D + (r16 & 1) * 8;
  const int tr_swz = dec_swz<ROWB>(tr_row);
  const int k_swz = dec_swz<ROWB>(r16);
  // unquantised V rows: lane (r16, kg) reads keys 4kg + r of head-dim column t * 16 + r16, one bf16
  // each, from logical chunk 2t + r16 / 8 of row 4kg + r, stored at chunk (2t + r16 / 8) ^ swz.
  // Its byte offset in the tile is v16_off[r] ^ (t << 5): the swizzle and t touch only bits 4 to
  // log2(ROWB) - 1, which the row offset, the lane's byte in the chunk and the tile's position in
  // LDS (a multiple of 16 rows) leave clear. Applying t as an XOR to the tile's own address keeps
  // one base per row instead of one hoisted address per (row, t) (NT x 4 registers at head_dim 256).
  uint32_t v16_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sw = dec_swz<ROWB>(4 * kg + r);
    v16_off[r] = (uint32_t)((4 * kg + r) * ROWB + (r16 & 7) * 2 + ((sw >> 1) << 5) + (((r16 >> 3) ^ (sw & 1)) << 4));
  }
  // byte offset, within a tile's 16 rows of a page, of this lane's 16-byte chunk in copy i:
  // LDS chunk q = 64 i + lane holds logical chunk (q % CPR) ^ dec_swz(row) of row q / CPR
  int dma_off[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int q = 64 * i + lane;
    dma_off[i] = (q / CPR) * ROWB + (((q % CPR) ^ dec_swz<ROWB>(q / CPR)) << 4);
  }

  // without a soft-cap, log2(e) folds into the logit scale
  const float xscale = CAP ? a.logit_scale : a.logit_scale * kLog2e;

  struct Pos { int k0, bi, r0; };
  auto advance = [&](Pos p) {
    p.k0 += STEP;
    p.r0 += STEP;
    if constexpr (GBS) {
      const int nb = small_quot(p.r0, a.inv_bs);  // r0 < block_size + STEP
      p.bi += nb;
      p.r0 -= nb * a.block_size;
    } else {
      while (p.r0 >= a.block_size) { p.r0 -= a.block_size; ++p.bi; }
    }
    return p;
  };
  // the wave's first tile of a segment and its tile count there (iterations it = w, w+4, ...)
  auto first_pos = [&](const DecSeg& sg, Pos& p) {
    const int it_base = (sg.k_lo / kTileKeys) * kTileKeys;
    const int n_iter = (sg.k_hi - it_base + kDecIterKeys - 1) / kDecIterKeys;
    p.k0 = it_base + wave * kDecIterKeys;
    p.bi = p.k0 / a.block_size;
    p.r0 = p.k0 - p.bi * a.block_size;
    return wave < n_iter ? (n_iter - wave + kDecWaves - 1) / kDecWaves : 0;
  };
  // ---- issue side: the wave's tile stream, walked ahead of the compute side
  int is_si = s_begin, is_left = 0, q_issued = 0, n_issued = 0;
  Pos is_p = {0, 0, 0};
  DecSeg is_sg = {};
  cptr<int32_t> is_bt = as_const(a.block_tables);
  const uint8_t* is_kv = a.cache;  // K page of the segment's KV head in block 0
  int32_t is_blk = 0;              // block-table entry of the next tile (read one tile ahead)
  i32x16 is_ent = {};              // GBS: entries of the 16 blocks from the next tile's first
  uint64_t ok_rows = 0;            // GBS: bits 16 (n & 3) ..: rows of tile n in blocks of the pool
  // the next tile's block-table entries (scalar loads; clamped to the sequence's table row); with
  // GBS and block_size >= 16 a tile spans at most two blocks, so two entries do
  auto fetch_blk = [&]() {
    if constexpr (GBS) {
      if (a.block_size >= kTileKeys) {
        is_ent[0] = is_bt[is_p.bi];
        is_ent[1] = is_bt[min(is_p.bi + 1, a.max_blocks - 1)];
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) is_ent[j] = is_bt[min(is_p.bi + j, a.max_blocks - 1)];
      }
    } else {
      is_blk = is_bt[is_p.bi];
    }
  };
  bool is_new = false;             // the next tile opens a segment: its Q rows go first
  uint32_t is_slot = 0;            // ring byte offset of the next tile
  uint64_t ok_bits = 0;            // bit (n & 63): tile n lies in a valid block
  // moves the cursor to this wave's first tile at or after segment si
  auto seek = [&](int si) {
    for (; si < s_end; ++si) {
      is_sg = load_const(as_const(a.segs) + si);
      is_left = first_pos(is_sg, is_p);
      if (is_left > 0) {
        is_si = si;
        is_new = true;
        is_bt = as_const(a.block_tables) + (int64_t)is_sg.seq * a.max_blocks;
        is_kv = a.cache + (int64_t)is_sg.kvh * a.page_bytes;
        fetch_blk();
        return;
      }
    }
    is_si = s_end;
    is_left = 0;
  };
  // GBS: the copies of the next tile row by row. Row t (key k0 + t) lies j = (r0 + t) / bs blocks
  // after the tile's first block, at row r0 + t - j bs; j < 16 as r0 < bs. An entry outside the
  // pool masks its rows (block 0 is read in their place).
  auto row_src = [&](int t, const uint8_t* base, int& rr, bool& ok) {
    const int n = is_p.r0 + t;
    int j;
    int32_t e;
    if (a.block_size >= kTileKeys) {  // (uniform) n < 2 block_size: the first or the next block
      j = n >= a.block_size ? 1 : 0;
      e = j ? is_ent[1] : is_ent[0];
    } else {
      j = small_quot(n, a.inv_bs);
      e = sel16(is_ent, j);
    }
    rr = n - j * a.block_size;
    ok = (uint32_t)e < (uint32_t)a.num_blocks;
    return base + (uint64_t)(ok ? (uint32_t)e : 0u) * (uint64_t)a.block_bytes;
  };
  auto issue_rows = [&]() {
    const uint32_t slot = ring_lds + is_slot;
    const int64_t voff = (int64_t)a.num_kv_heads * a.page_bytes;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int q = 64 * i + lane, t = q / CPR;
      int rr;
      bool ok;
      const uint8_t* pg = row_src(t, is_kv, rr, ok);
      const uint8_t* src = pg + (int64_t)rr * ROWB + ((((q % CPR) ^ dec_swz<ROWB>(t))) << 4);
      dma16_to_lds(src, slot + (uint32_t)(1024 * i));
      dma16_to_lds(src + voff, slot + (uint32_t)(TB + 1024 * i));
    }
    {
      int rr;
      bool ok;
      row_src(lane & 15, is_kv, rr, ok);
      const uint32_t rows = (uint32_t)__builtin_amdgcn_ballot_w64(ok && lane < 16) & 0xFFFFu;
      const int sh = 16 * (n_issued & 3);
      ok_rows = (ok_rows & ~(0xFFFFull << sh)) | ((uint64_t)rows << sh);
    }
    if constexpr (PTH) {
      // lanes 0..15: the K scales of rows 0..15, lanes 16..31: the V scales
      int rr;
      bool ok;
      const uint8_t* pg = row_src(lane & 15, is_kv + ((lane & 16) ? voff : 0), rr, ok);
      if (lane < 32) dma4_to_lds(pg + (int64_t)a.block_size * D + 4 * rr, slot + (uint32_t)(2 * TB));
    }
    if constexpr (PG) {
      // [K: 16 rows x NG][V: 16 rows x NG] floats, 64 per copy
#pragma unroll
      for (int c = 0; c < SCC; ++c) {
        const int idx = 64 * c + lane;
        const int kv = idx / (16 * NG), rem = idx % (16 * NG);
        const int t = rem / NG, g = rem % NG;
        int rr;
        bool ok;
        const uint8_t* pg = row_src(t, is_kv + (kv ? voff : 0), rr, ok);
        if (idx < 32 * NG) dma4_to_lds(pg + (int64_t)a.block_size * D + 4 * ((int64_t)rr * NG + g), slot + (uint32_t)(2 * TB + 256 * c));
      }
    }
  };
  // issues the next tile if its ring slot (and, for a new segment, a Q slot) is free
  auto issue_next = [&](int n_done, int q_read) {
    if (is_left <= 0 || n_issued - n_done >= NS) return;
    if (is_new) {
      if (q_issued - q_read >= NQ) return;
      // the segment's q rows, contiguous: [nheads][D] bf16 into Q slot q_issued % NQ
      const int nbytes = is_sg.nheads * D * 2;
      const uint8_t* src = (const uint8_t*)(a.q + ((int64_t)is_sg.q_tok * a.num_q_heads + is_sg.kvh * a.group + is_sg.head0) * D);
      const uint32_t dst = q_lds + (uint32_t)((q_issued % NQ) * QB);
      for (int o = 0; o < nbytes; o += 1024)
        if (o + lane * 16 < nbytes) dma16_to_lds(src + o + lane * 16, dst + (uint32_t)o);
      ++q_issued;
      is_new = false;
    }
    if constexpr (GBS) {
      issue_rows();
    } else {
    // an entry outside the pool masks its tile instead of reading outside the cache
    const bool ok = (uint32_t)is_blk < (uint32_t)a.num_blocks;
    ok_bits = (ok_bits & ~(1ull << (n_issued & 63))) | ((uint64_t)ok << (n_issued & 63));
    const uint8_t* kpage = is_kv + (uint64_t)(ok ? (uint32_t)is_blk : 0u) * (uint64_t)a.block_bytes +
                           (int64_t)is_p.r0 * ROWB;
    const uint8_t* vpage = kpage + (int64_t)a.num_kv_heads * a.page_bytes;
    const uint32_t slot = ring_lds + is_slot;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      dma16_to_lds(kpage + dma_off[i], slot + (uint32_t)(1024 * i));
      dma16_to_lds(vpage + dma_off[i], slot + (uint32_t)(TB + 1024 * i));
    }
    if constexpr (PTH) {
      // lanes 0..3: the 16 K scales, lanes 4..7: the 16 V scales
      const uint8_t* sp = ((lane & 4) ? vpage : kpage) + (int64_t)(a.block_size - is_p.r0) * D + 4 * (is_p.r0 + 4 * (lane & 3));
      if (lane < 8) dma16_to_lds(sp, slot + (uint32_t)(2 * TB));
    }
    if constexpr (PG) {
      // the tile's 16 x NG group scales of K (lanes 0 .. 4NG-1), then of V (lanes 4NG .. 8NG-1)
      const int sl = lane % (4 * NG);
      const uint8_t* sp = (lane >= 4 * NG ? vpage : kpage) + (int64_t)(a.block_size - is_p.r0) * D +
                          4 * (int64_t)is_p.r0 * NG + 16 * sl;
      if (lane < 8 * NG) dma16_to_lds(sp, slot + (uint32_t)(2 * TB));
    }
    }
    ++n_issued;
    is_slot = is_slot + SLOT == NS * SLOT ? 0u : is_slot + SLOT;
    if (--is_left > 0) {
      is_p = advance(is_p);
      fetch_blk();  // needed only at the next issue: its latency hides behind a tile
    } else {
      seek(is_si + 1);
    }
  };

  // the work-group's first segment comes from its own record (loaded at the start, beside the
  // segment range), so the first copies do not wait on the range and then the segment; every
  // work-group has at least one segment
  is_sg = first_sg;
  is_left = first_pos(is_sg, is_p);
  if (is_left > 0) {
    is_si = s_begin;
    is_new = true;
    is_bt = as_const(a.block_tables) + (int64_t)is_sg.seq * a.max_blocks;
    is_kv = a.cache + (int64_t)is_sg.kvh * a.page_bytes;
    fetch_blk();
  } else {
    seek(s_begin + 1);
  }
#pragma unroll
  for (int k = 0; k < NS; ++k) issue_next(0, 0);

  // ---- compute side
  int n_done = 0, q_read = 0;
  uint32_t c_slot = 0;
  bf16x8 qb[QS];
  for (int si = s_begin; si < s_end; ++si) {
    const DecSeg sg = load_const(as_const(a.segs) + si);
    const bool head_ok = r16 < sg.nheads;
    // ALiBi: slope of this lane's head (log2 domain) and the query's position L - 1
    float slope2 = 0.0f;
    int qpos = 0;
    if (a.alibi) {
      qpos = as_const(a.seq_lens)[sg.seq] - 1;
      slope2 = head_ok ? a.alibi[sg.kvh * a.group + sg.head0 + r16] * kLog2e : 0.0f;
    }
    Pos pc0;
    const int n_my = first_pos(sg, pc0);
    int ck0 = pc0.k0;  // first key of the wave's next tile

    float m = -INFINITY;  // reference max (log2 domain) of this lane's head
    float l = 0.0f;       // sum of this lane's probabilities relative to m
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One tile's scores (keys k0 + 4 kg + r of head r16, log2 domain, masked) and its V operands,
    // read from the ring slot at `kl`.
    struct TileS {
      float x[4];
      i32x2 vw[EB == 1 ? NT / 2 : 1];
      uint32_t vb[EB == 2 ? NT : 1][2];
      float4 vs;
      uint32_t vmask;
      bool full;
    };
    // rows_ok: bit t set when row t of the tile lies in a block of the pool (without GBS a tile
    // lies in one block: a flag)
    using RowMask = std::conditional_t<GBS, uint32_t, bool>;
    auto score = [&](const uint8_t* kl, int k0, RowMask rows_ok, TileS& t) {
      const uint8_t* vl = kl + TB;
      // ---- S^T = K * Q^T: lane holds keys k0 + 4kg + r of head r16
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      if constexpr (PG) {
        // per group: MFMA step st takes depth 32*st + 8*kg + 0..7 (group st) from K, exactly
        // widened; its product is scaled per key by that key's group scale, in fp32
        const float* ksr = (const float*)(kl + 2 * TB) + (4 * kg) * NG;
#pragma unroll
        for (int st = 0; st < QS; ++st) {
          const uint2 w = *(const uint2*)(kl + r16 * ROWB + (((2 * st + (kg >> 1)) ^ k_swz) << 4) + 8 * (kg & 1));
          const f32x4 sg = mfma16x16x32(widen8<DT>(w.x, w.y), qb[st], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) s[r] += ksr[r * NG + st] * sg[r];
        }
      } else if constexpr (EB == 1) {
#pragma unroll
        for (int c2 = 0; c2 < QS / 2; ++c2) {
          const uint4 w = *(const uint4*)(kl + r16 * ROWB + (((kg * (QS / 2) + c2) ^ k_swz) << 4));
          s = mfma16x16x32(widen8<DT>(w.x, w.y), qb[2 * c2], s);
          s = mfma16x16x32(widen8<DT>(w.z, w.w), qb[2 * c2 + 1], s);
        }
      } else {
        // bf16 rows: each 16-byte chunk is one operand (depth kg * D/4 + 8 st .. +7)
#pragma unroll
        for (int st = 0; st < QS; ++st)
          s = mfma16x16x32(*(const bf16x8*)(kl + r16 * ROWB + (((kg * QS + st) ^ k_swz) << 4)), qb[st], s);
      }
      // V^T operands: transposed reads issued now, used after the softmax
      if constexpr (EB == 1) {
#pragma unroll
        for (int t2 = 0; t2 < NT / 2; ++t2) t.vw[t2] = lds_read_tr8(vl + tr_base + (((2 * t2 + tr_hi) ^ tr_swz) << 4));
      } else {
        static_assert(TB % (16 * ROWB) == 0 && SLOT % (16 * ROWB) == 0, "V tiles start at multiples of 16 rows");
        const uint32_t vo = (uint32_t)(vl - smem);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          uint32_t e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) e[r] = *(const uint16_t*)(smem + ((vo + v16_off[r]) ^ (uint32_t)(tt << 5)));
          t.vb[tt][0] = e[0] | (e[1] << 16);
          t.vb[tt][1] = e[2] | (e[3] << 16);
        }
      }
      float4 ks;
      if constexpr (PTH) {
        ks = *(const float4*)(kl + 2 * TB + 16 * kg);
        t.vs = *(const float4*)(kl + 2 * TB + 64 + 16 * kg);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) t.x[r] = s[r] * xscale;
      if constexpr (PTH) {
        t.x[0] *= ks.x; t.x[1] *= ks.y; t.x[2] *= ks.z; t.x[3] *= ks.w;
      }
      if constexpr (CAP) {
#pragma unroll
        for (int r = 0; r < 4; ++r) t.x[r] = a.softcap * kLog2e * tanh_via_exp2(t.x[r] * a.inv_softcap);
      }
      if (a.alibi) {
        // + slope * (key - position), after the soft-cap
        const int base = k0 + 4 * kg - qpos;
#pragma unroll
        for (int r = 0; r < 4; ++r) t.x[r] += slope2 * (float)(base + r);
      }
      // masking is needed only on the segment's edge tiles (and tiles of an invalid block); rows
      // outside the range may hold unwritten bytes: their logits are replaced, their V codes
      // masked to zero and (per token-head) their scales replaced, so no NaN reaches the sums
      t.full = (GBS ? (uint32_t)rows_ok == 0xFFFFu : (bool)rows_ok) && k0 >= sg.k_lo && k0 + kTileKeys <= sg.k_hi;
      t.vmask = 0xFFFFFFFFu;
      if (!t.full) {
        t.vmask = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 4 * kg + r;
          const bool row_ok = GBS ? (((uint32_t)rows_ok >> (4 * kg + r)) & 1) != 0 : (bool)rows_ok;
          const bool kok = row_ok && key >= sg.k_lo && key < sg.k_hi;
          t.x[r] = kok ? t.x[r] : -INFINITY;
          if (kok) t.vmask |= 0xFFu << (8 * r);
        }
      }
    };
    // the probabilities of one tile (relative to m_use) into l and its PV product into acc
    auto accumulate = [&](const uint8_t* kl, TileS& t, float m_use) {
      float p4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p4[r] = fast_exp2(t.x[r] - m_use);
      l += (p4[0] + p4[1]) + (p4[2] + p4[3]);
      const uint32_t vmask = t.vmask;
      if constexpr (PTH) {
        float4 vs = t.vs;
        if (!t.full) {
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
      // ---- O^T[d][head] += V^T[d][keys] P^T[keys][head]
      if constexpr (PG) {
        // per group: head-dim tiles 2g, 2g+1 form group g; its P^T operand carries the keys' V
        // scales of that group (masked keys select 0: their scale slots may be unwritten)
        const float* vsg = (const float*)(kl + 2 * TB) + 16 * NG + (4 * kg) * NG;
#pragma unroll
        for (int t2 = 0; t2 < NT / 2; ++t2) {
          bf16x4 pg;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool kok = (vmask >> (8 * r)) & 1;
            pg[r] = (__bf16)(kok ? p4[r] * vsg[r * NG + t2] : 0.0f);
          }
          acc[2 * t2] = mfma16x16x16(widen4v<DT>((uint32_t)t.vw[t2].x & vmask), pg, acc[2 * t2]);
          acc[2 * t2 + 1] = mfma16x16x16(widen4v<DT>((uint32_t)t.vw[t2].y & vmask), pg, acc[2 * t2 + 1]);
        }
      } else if constexpr (EB == 1) {
#pragma unroll
        for (int t2 = 0; t2 < NT / 2; ++t2) {
          acc[2 * t2] = mfma16x16x16(widen4v<DT>((uint32_t)t.vw[t2].x & vmask), pb, acc[2 * t2]);
          acc[2 * t2 + 1] = mfma16x16x16(widen4v<DT>((uint32_t)t.vw[t2].y & vmask), pb, acc[2 * t2 + 1]);
        }
      } else {
        // masked keys: their (possibly unwritten) bf16 values are zeroed like the codes above
        const uint32_t m01 = ((vmask & 0xFFu) ? 0xFFFFu : 0u) | ((vmask & 0xFF00u) ? 0xFFFF0000u : 0u);
        const uint32_t m23 = ((vmask & 0xFF0000u) ? 0xFFFFu : 0u) | ((vmask & 0xFF000000u) ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const uint2 u = make_uint2(t.vb[tt][0] & m01, t.vb[tt][1] & m23);
          acc[tt] = mfma16x16x16(__builtin_bit_cast(bf16x4, u), pb, acc[tt]);
        }
      }
    };
    // lazy rescaling: the reference max moves (and O, l are rescaled) only when some head's max
    // exceeds it by more than 2^8, so probabilities stay <= 256 and the common case leaves the
    // accumulators alone; returns the reference the probabilities are taken against
    auto rescale_to = [&](float mx) {
      if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.0f : m_new));
        l *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] *= alpha;
        m = m_new;
      }
      return m == -INFINITY ? 0.0f : m;
    };
    auto load_q = [&]() {
      // Q^T operand: lane (column head r16, group kg) holds q[head][kg*D/4 + 8*st + 0..7]
      // (per group: q[head][32*st + 8*kg + 0..7], so that MFMA step st covers scale group st)
      const uint8_t* qp = qslots + (q_read % NQ) * QB + r16 * (D * 2) + (PG ? kg * 16 : kg * (D / 2));
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        uint4 u = *(const uint4*)(qp + st * (PG ? 64 : 16));
        if (!head_ok) u = make_uint4(0, 0, 0, 0);
        qb[st] = __builtin_bit_cast(bf16x8, u);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      ++q_read;
      issue_next(n_done, q_read);  // a copy held back for want of a Q slot
    };
    auto next_slot = [&](uint32_t c) { return c + SLOT == NS * SLOT ? 0u : c + SLOT; };
    auto tile_rows = [&](int n) -> RowMask {
      if constexpr (GBS) return (uint32_t)(ok_rows >> (16 * (n & 3))) & 0xFFFFu;
      else return (ok_bits >> (n & 63)) & 1;
    };
    // two of the wave's tiles per iteration (one reduction and rescale check for both) where the
    // ring holds at least three tiles (so one stays in flight while a pair is computed), then the
    // rest one at a time
    int k = 0;
    for (; NS >= 3 && k + 1 < n_my; k += 2) {
      // both tiles' copies are done once only later tiles' copies are outstanding
      wait_tiles_ahead<IPT, NS>(n_issued - n_done - 2);
      if (k == 0) load_q();
      const uint8_t* kl0 = ring + c_slot;
      const uint8_t* kl1 = ring + next_slot(c_slot);
      TileS t0, t1;
      score(kl0, ck0, tile_rows(n_done), t0);
      score(kl1, ck0 + STEP, tile_rows(n_done + 1), t1);
      const float mx = max_over_rows(fmaxf(fmaxf(fmaxf(t0.x[0], t0.x[1]), fmaxf(t0.x[2], t0.x[3])),
                                           fmaxf(fmaxf(t1.x[0], t1.x[1]), fmaxf(t1.x[2], t1.x[3]))));
      const float m_use = rescale_to(mx);
      accumulate(kl0, t0, m_use);
      accumulate(kl1, t1, m_use);
      n_done += 2;
      c_slot = next_slot(next_slot(c_slot));
      ck0 += 2 * STEP;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_next(n_done, q_read);  // into the slots these tiles used: every read of them is complete
      issue_next(n_done, q_read);
    }
    for (; k < n_my; ++k) {
      wait_tiles_ahead<IPT, NS>(n_issued - n_done - 1);
      if (k == 0) load_q();
      const uint8_t* kl0 = ring + c_slot;
      TileS t0;
      score(kl0, ck0, tile_rows(n_done), t0);
      const float m_use = rescale_to(max_over_rows(fmaxf(fmaxf(t0.x[0], t0.x[1]), fmaxf(t0.x[2], t0.x[3]))));
      accumulate(kl0, t0, m_use);
      ++n_done;
      c_slot = next_slot(c_slot);
      ck0 += STEP;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_next(n_done, q_read);
    }

    // ---- hand (O, m, l) to the fetching wave, which merges the four waves and writes the
    // result while these waves go on with the next segment
    l = sum_over_rows(l);
    block_sync_lds();  // the fetching wave has read the previous segment's values
    if (r16 < gh) {
      float* dst = mg + (wave * gh + r16) * merge_stride(D);
#pragma unroll
      for (int t = 0; t < NT; ++t) *(f32x4*)(dst + t * 16 + 4 * kg) = acc[t];
      if (kg == 0) { dst[D] = m; dst[D + 1] = l; }
    }
    block_sync_lds();
  }
  // every copy this wave issued has landed before it exits
  wait_vmcnt(0);
}

// Merge of partial results (split decode ranges, split prefill runs): one wave per (item, head).
// M = max_s m_s; O = sum_s 2^(m_s - M) O_s / (sum_s 2^(m_s - M) l_s [+ 2^(sink - M)]).
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const CombItem* items, const float* scratch, uint16_t* out,
                                                     int32_t num_q_heads, int32_t group, int64_t num_slots,
                                                     const float* sinks) {
  const CombItem it = load_const(as_const(items) + blockIdx.x);
  const int h = blockIdx.y;
  if (h >= it.nheads) return;
  const int lane = threadIdx.x;
  const int P = it.num_parts;
  const float* ml = scratch + num_slots * D;
  auto slot = [&](int s) { return (int64_t)it.first_slot + (int64_t)s * it.part_stride + h; };
  constexpr int PER = D / 64;
  // the rows of the first PRE parts are loaded at once with the (m, l) values: they do not depend
  // on the weights, so their latency overlaps the max and sum reductions
  constexpr int PRE = 8;
  const int npre = min(P, PRE);
  float vp[PRE][PER];
#pragma unroll
  for (int u = 0; u < PRE; ++u)
    if (u < npre)
#pragma unroll
      for (int j = 0; j < PER; ++j) vp[u][j] = scratch[slot(u) * D + lane + 64 * j];
  // (m, l) of the parts: lane s takes parts s, s + 64, ..., so their loads are all in flight at once
  float M = -INFINITY;
  for (int s = lane; s < P; s += 64) M = fmaxf(M, ml[slot(s) * 2]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, shfl_xor_f(M, k));
  const float M_use = M == -INFINITY ? 0.0f : M;
  float L = 0.0f;
  for (int s = lane; s < P; s += 64) L += fast_exp2(ml[slot(s) * 2] - M_use) * ml[slot(s) * 2 + 1];
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) L += shfl_xor_f(L, k);
  float o[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] = 0.0f;
  for (int s0 = 0; s0 < P; s0 += 64) {
    // weight of part s0 + lane, broadcast part by part; four parts' rows loaded before any is summed
    const float fl = s0 + lane < P ? fast_exp2(ml[slot(s0 + lane) * 2] - M_use) : 0.0f;
    const int n = min(64, P - s0);
    int s = 0;
    if (s0 == 0) {
#pragma unroll
      for (int u = 0; u < PRE; ++u)
        if (u < npre) {
          const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), u));
#pragma unroll
          for (int j = 0; j < PER; ++j) o[j] += f * vp[u][j];
        }
      s = npre;
    }
    for (; s + 4 <= n; s += 4) {
      float v[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < PER; ++j) v[u][j] = scratch[slot(s0 + s + u) * D + lane + 64 * j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), s + u));
#pragma unroll
        for (int j = 0; j < PER; ++j) o[j] += f * v[u][j];
      }
    }
    for (; s < n; ++s) {
      const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), s));
#pragma unroll
      for (int j = 0; j < PER; ++j) o[j] += f * scratch[slot(s0 + s) * D + lane + 64 * j];
    }
  }
  const int hq = it.kvh * group + it.head0 + h;
  float fs = 1.0f;
  if (sinks) {
    // the sink logit joins the normaliser (log2 domain), relative to the same reference as o and L
    const float s2 = sinks[hq] * kLog2e;
    const float Mx = fmaxf(M_use, s2);
    fs = fast_exp2(M_use - Mx);
    L = L * fs + fast_exp2(s2 - Mx);
  }
  const float inv = L > 0.0f ? fs / L : 0.0f;  // no key in any part and no sink: 0
  uint16_t* op = out + ((int64_t)it.q_tok * num_q_heads + hq) * D;
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
  d.first = (const DecSeg*)(a.meta_dev + h.off_dec_first);
  d.scratch = a.scratch;
  d.out = a.out;
  d.page_bytes = a.page_bytes;
  d.block_bytes = a.block_bytes;
  d.block_size = a.block_size;
  d.inv_bs = 1.0f / (float)a.block_size;
  d.num_kv_heads = a.num_kv_heads;
  d.num_q_heads = a.num_q_heads;
  d.group = a.group;
  d.max_blocks = a.max_blocks_per_seq;
  d.group_heads = h.group_heads;
  d.num_blocks = h.num_blocks;
  d.num_slots = h.num_slots;
  d.logit_scale = MODE == AQP_SCALE_PER_TENSOR ? a.sm_scale * a.k_scale : a.sm_scale;
  d.softcap = a.softcap;
  d.inv_softcap = a.softcap > 0.0f ? 1.0f / a.softcap : 0.0f;
  d.v_scale = MODE == AQP_SCALE_PER_TENSOR ? a.v_scale : 1.0f;
  d.seq_lens = (const int32_t*)(a.meta_dev + h.off_seq_lens);
  d.alibi = a.alibi_slopes;
  d.sinks = a.sinks;
  const dim3 grid(h.num_dec_wgs), block((kDecWaves + 1) * 64);
  if (a.block_size % kTileKeys != 0) {
    if (a.softcap > 0.0f)
      hipLaunchKernelGGL((decode_kernel<D, DT, MODE, true, true>), grid, block, h.dec_lds_bytes, st, d);
    else
      hipLaunchKernelGGL((decode_kernel<D, DT, MODE, false, true>), grid, block, h.dec_lds_bytes, st, d);
  } else if (a.softcap > 0.0f) {
    hipLaunchKernelGGL((decode_kernel<D, DT, MODE, true, false>), grid, block, h.dec_lds_bytes, st, d);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, DT, MODE, false, false>), grid, block, h.dec_lds_bytes, st, d);
  }
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
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_AUTO) return dec_d<AQP_KV_AUTO, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E4M3) return dec_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E5M2) return dec_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_INT8) return dec_d<AQP_KV_INT8, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E4M3) return dec_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_INT8) return dec_d<AQP_KV_INT8, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E5M2) return dec_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_INT8) return dec_d<AQP_KV_INT8, AQP_SCALE_PER_GROUP>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_FP8_E4M3) return dec_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_GROUP>(a, st);
  if (mode == AQP_SCALE_PER_GROUP && dtype == AQP_KV_FP8_E5M2) return dec_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_GROUP>(a, st);
  set_error("aqp_paged_attention: dtype %d with scale mode %d is not built", dtype, mode);
  return AQP_ERR_UNSUPPORTED;
}

int launch_combine(const AttnArgs& a, int32_t first, int32_t count, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const SchedHeader& h = *a.hdr;
  const CombItem* items = (const CombItem*)(a.meta_dev + h.off_comb) + first;
  dim3 grid(count, (uint32_t)h.comb_heads);
  switch (a.head_dim) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(64), 0, st, items, a.scratch, a.out, a.num_q_heads, a.group, h.num_slots, a.sinks); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(64), 0, st, items, a.scratch, a.out, a.num_q_heads, a.group, h.num_slots, a.sinks); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(64), 0, st, items, a.scratch, a.out, a.num_q_heads, a.group, h.num_slots, a.sinks); break;
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
