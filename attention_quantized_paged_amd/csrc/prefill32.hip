// Prefill attention on 32x32x16 bf16 MFMAs, for caches of one-byte codes with per-tensor or
// per-token-head scales (the pairs the pages name: fp8 e4m3 / e5m2 per tensor, the "CPU backend
// adds FP8 KV-cache quantisation" page, vllm PR 39445; int8 / fp8 per token-head, the
// "Per-token-head INT8/FP8 KV quantisation for Triton" page, vllm PR 38378, and the two other
// codec pairs). Same method as the other attention kernels: the dequantise step fused into the
// two tile products (PR 39445 page, Implementation item 2), online softmax, folded scales; the
// large-prefill shape of the "Fix CPU FP8 attention scheduler scratch sizing" page (vllm PR
// 50194, Code excerpt: head_size 256, block_size 2176) is the one it is tuned on.
//
// gfx950 mapping. A work-group takes one schedule item: up to 32 * WAVES query rows (token-major:
// row r is token r / nheads, q head r % nheads, so all rows share the K/V tiles); each wave owns 32
// rows, the 32 columns of its MFMA tiles. Per step of 32 keys:
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, one dependent chain over the head dimension: A = 32
//                   keys x 16 depth from a bf16 image of the step's keys (widened once per
//                   work-group, a quarter per wave, one step ahead; 1 KB operand blocks read as 64
//                   lanes x 16 bytes); B = Q^T, in registers for the whole item. Lane l holds row
//                   l % 32 and keys 8 (i / 4) + 4 (l / 32) + i % 4 of its 16 accumulators i.
//   softmax         per row over the lane's 16 keys and its partner lane l ^ 32 (one lane swap);
//                   exp2 domain, lazy rescaling; per-token-head scales read from the ring stage
//                   (the K scales staged times the logit scale).
//   O^T += V^T P^T  A = V^T from a bf16 image of the step's values (widened once per work-group,
//                   64 lanes x 16 bytes per 1 KB operand block, in exactly the key order the
//                   probabilities sit in: lane half h of 16-key chunk c holds keys
//                   16 c + 8 (j / 4) + 4 h + j % 4, j = 0..7); B = the probabilities where S^T left
//                   them, rounded to bf16.
// The codes of 32 keys of K and V (and their per-token-head scales) go from HBM through registers
// (16-byte loads, one iteration ahead of their LDS write) into a 4-stage LDS ring (16-byte chunks,
// XOR-swizzled so that both the 16-row K reads and the 8-row transposed V reads hit distinct
// banks); one barrier per step orders the ring and the images. Register staging rather than the
// direct global -> LDS copy: the compiler counts these loads and waits for exactly the ones a store
// needs, while hand-issued copies are invisible to its counting, so any load it issues itself
// (spill reloads, table reads) gets a vmcnt(0) wait that drains every copy in flight. The
// block-table entries of the item's tiles are gathered 64 tiles at a time into a small LDS table
// and held one per lane.
#include <type_traits>

#include "device_common.h"

namespace aqp {

struct Pf32Args {
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
  uint32_t bs_magic;   // key / block_size = div_invariant(key, bs_magic, bs_shift)
  int32_t bs_shift;
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Stored 16-byte chunk of logical chunk c in staged row `row` (rows of D bytes): c ^ pf32_swz(row).
// m is the row's index among the rows that share a 256-byte line position; the permutation is
// chosen so that (a) any 16 consecutive rows read at one logical chunk fall on 16 distinct
// 16-byte bank groups (the K operand reads), and (b) the 8 rows of one lane half of a 16-key
// chunk (keys 4h + {0..3, 8..11}), read at two adjacent logical chunks, do too (the transposed V
// reads): within those rows the swizzle takes 8 distinct values of one parity.
template <int D>
__device__ __forceinline__ int pf32_swz(int row) {
  if constexpr (D >= 256) {
    const int m = row & 15;
    return ((m & 3) << 1) | (m & 8) | ((m >> 2) & 1);
  } else if constexpr (D == 128) {
    const int m = (row >> 1) & 7;
    return ((m & 1) << 1) | (m & 4) | ((m >> 1) & 1);
  } else {
    return (row >> 2) & 3;
  }
}

// Widen 16 codes (one 16-byte read) into two MFMA operands of 8 bf16 each.
template <int DT>
__device__ __forceinline__ void widen16(uint4 c, bf16x8& lo, bf16x8& hi) {
  lo = widen8<DT>(c.x, c.y);
  hi = widen8<DT>(c.z, c.w);
}

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<0>{}), ..., f(IC<N - 1>{}): a loop whose index is a constant in each body
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<N, I + 1>(f);
  }
}

// Reference to one of two objects chosen at compile time (the ping-pong buffers of the step loop).
template <int I, typename T>
__device__ __forceinline__ T& pick(T& a, T& b) {
  if constexpr (I == 0) return a;
  else return b;
}

template <int D, int DT, int MODE, bool CAP, bool ALIBI, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(pf32_waves_per_simd(D, MODE))))
void prefill32_kernel(Pf32Args a) {
  constexpr int KT = kPfKvTile;                    // keys per step
  static_assert(KT == 32, "one 32x32 S tile per step");
  constexpr int NS = kPf32Stages;                  // LDS ring stages
  static_assert(NS == 4, "the step loop is unrolled over the four ring stages");
  constexpr int ROWB = D;                          // bytes of one staged key row (one-byte codes)
  constexpr int CPR = ROWB / 16;                   // 16-byte chunks per row
  constexpr int PTH = MODE == AQP_SCALE_PER_TOKEN_HEAD ? 1 : 0;
  constexpr int SCB = PTH ? 2 * KT * 4 : 0;        // scale bytes of a step: K then V
  constexpr int STAGE = pf32_stage_bytes(D, MODE);
  static_assert(STAGE == 2 * KT * ROWB + SCB, "stage layout");
  constexpr int KVI = KT * CPR / 64;               // 1 KB copies per K (or V) step
  constexpr int IPW = 2 * KVI / WAVES;             // K+V copies per wave per step
  static_assert(IPW >= 1 && (2 * KVI) % WAVES == 0, "copies must split evenly over the waves");
  constexpr int RPC = 1024 / ROWB;                 // key rows per copy
  constexpr int QC = D / 16;                       // 16-deep chunks of the QK^T product
  constexpr int NDT = D / 32;                      // 32-wide head-dim tiles of O
  constexpr int VBLK = 2 * NDT;                    // V image blocks: [dim tile][16-key chunk]
  constexpr int VB_PW = VBLK / WAVES;              // V blocks each wave widens per step
  static_assert(VB_PW >= 1 && VBLK % WAVES == 0, "V blocks must split evenly over the waves");
  constexpr int VIMG = VBLK * 1024;                // one step's V image (and one step's K image)
  static_assert(QC * 1024 == VIMG, "K and V images are the same size");
  constexpr int KIM = 2 * VIMG;                    // the two K images follow the two V images
  constexpr int RB = 4 * VIMG;                     // then the ring
  constexpr int TBL = RB + NS * STAGE;             // then the tile tables: [batch parity][wave][64]
  static_assert(WAVES <= 4 && TBL + kPf32TableBytes == pf32_lds_bytes(D, MODE), "LDS layout");
  static_assert((NS - 1) * STAGE + 1024 < 65536 && 4 * VIMG <= 65536, "constant LDS offsets fit the 16-bit offset field");
  constexpr int KU = 4 * D / (64 * WAVES);         // 8-code units of a step's K image each lane widens
  static_assert(KU >= 1 && KU <= 8 && (KU == 1 || KU % 2 == 0) && QC % KU == 0, "K image units per lane");
  constexpr int NSL = QC;                          // slices of a step: one S chunk and one PV block each
  static_assert(QC == 2 * NDT, "as many S chunks as PV blocks");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r32 = lane & 31;  // the lane's row within the wave (MFMA column)
  const int hh = lane >> 5;   // lane half
  const PfItem it = load_const(as_const(a.items) + blockIdx.x);
  if (it.q_hi <= it.q_lo) return;  // an empty item (launch-order padding)
  const int G = a.group;
  const int nh = it.nheads;
  const int ntok = it.q_hi - it.q_lo;
  const cptr<int32_t> bt = as_const(a.block_tables) + (int64_t)it.seq * a.max_blocks;
  const uint8_t* kbase = a.cache + (int64_t)it.kvh * a.page_bytes;
  const uint8_t* vbase = a.cache + (int64_t)(a.num_kv_heads + it.kvh) * a.page_bytes;

  // ---- this lane's row
  const int row = wave * 32 + r32;
  const int tl = row / nh;
  const int g_in = row - tl * nh;
  const bool row_ok = tl < ntok;
  const int tq = it.q_lo + (row_ok ? tl : 0);
  const int pos = it.L - it.ql + tq;  // position of the row's query
  const int hq = it.kvh * G + it.head0 + g_in;
  int hi_r = it.causal ? pos + 1 : it.L;
  int lo_r = (a.window > 0 && pos - a.window + 1 > 0) ? pos - a.window + 1 : 0;
  lo_r = max(lo_r, it.split_lo);  // a run of a split item sees only its own keys
  hi_r = min(hi_r, it.split_hi);
  if (!row_ok) { lo_r = 0; hi_r = 0; }
  const float slope2 = ALIBI ? a.alibi[hq] * kLog2e : 0.0f;
  const float sink2 = a.sinks ? a.sinks[hq] * kLog2e : -INFINITY;
  const int64_t orow = ((int64_t)(it.q_start + tq) * a.num_q_heads + hq) * D;
  // Q^T operands: chunk c of lane half h is depth h * D/2 + 8 c .. + 7 (the K operands below read
  // the same depths), so each lane holds one contiguous half of its row. (Loaded in the prologue
  // after the first steps' key/value loads: the wait for the block-table gather then does not
  // wait for the item's Q rows too, and their transfer overlaps the key/value loads.)
  bf16x8 qb[QC];
  auto load_q = [&]() {
    const uint16_t* qp = a.q + orow + hh * (D / 2);
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      uint4 u = *(const uint4*)(qp + 8 * c);
      if (!row_ok) u = make_uint4(0, 0, 0, 0);
      qb[c] = __builtin_bit_cast(bf16x8, u);
      // (kept in the matrix accumulation registers, which matrix instructions read as operands: the
      // ordinary registers are the scarcer ones here)
      if constexpr (D >= 256) asm volatile("" : "+a"(qb[c]));
    }
  };
  // keys visible to every row of the wave: [vis_lo, vis_hi)
  const int tw0 = min(ntok - 1, (wave * 32) / nh);
  const int tw1 = min(ntok - 1, (wave * 32 + 31) / nh);
  const bool wave_rows_full = (wave * 32 + 31) / nh < ntok;
  const int pw0 = it.L - it.ql + it.q_lo + tw0, pw1 = it.L - it.ql + it.q_lo + tw1;
  const int vis_hi = min(it.causal ? pw0 + 1 : it.L, it.split_hi);
  const int vis_lo = max((a.window > 0 && pw1 - a.window + 1 > 0) ? pw1 - a.window + 1 : 0, it.split_lo);
  // key range of the item: its first token's window start (16-aligned) .. its last token's end
  const int p_first = it.L - it.ql + it.q_lo;
  const int k_first = (a.window > 0 && p_first - a.window + 1 > 0) ? p_first - a.window + 1 : 0;
  const int k_begin = max((k_first / kTileKeys) * kTileKeys, it.split_lo);  // (split_lo: a step boundary)
  const int k_end = min(it.k_hi_max, it.split_hi);
  const int n_steps = (k_end - k_begin + KT - 1) / KT;
  const float xscale = CAP ? a.logit_scale : a.logit_scale * kLog2e;
  const int last_tile = ((it.L - 1) / kTileKeys) * kTileKeys;  // first key of the tile holding key L-1
  // steps s whose keys k_begin + 32 s .. + 31 every row of the wave sees and that end by key L:
  // f_lo <= s <= f_hi (their tiles must also be present to run unmasked)
  const int f_lo = vis_lo <= k_begin ? 0 : (vis_lo - k_begin + KT - 1) / KT;
  const int f_lim = min(vis_hi, it.L) - KT - k_begin;
  const int f_hi = wave_rows_full && f_lim >= 0 ? f_lim / KT : -1;

  // ---- copies of one step into its ring stage. Copy ii = wave * IPW + j (0 .. 2 KVI - 1) fills LDS
  // bytes 1024 ii .. of the stage: 64 chunks of K (ii < KVI) or V, lane l taking chunk
  // q = 64 (ii % KVI) + l of the step, key row q / CPR, stored position q % CPR, which holds logical
  // chunk (q % CPR) ^ swz(row). The TPC = 16 / RPC copies of a 16-key tile read it at one tile base
  // (wave-uniform) plus a per-lane offset fixed for the kernel and their position in the tile
  // (1 KB apart, an instruction offset that applies to the LDS side too): with k = ii % KVI the lane
  // offset is a lane part XOR a part of k that only flips chunk-index bits (the swizzle of row
  // 16-tile position m takes its copy-dependent bits from k).
  constexpr int TPC = 16 / RPC;                    // copies per 16-key tile
  static_assert(IPW % TPC == 0, "a wave copies whole tiles");
  uint32_t cp_v[IPW];
  {
    const int rr = lane / CPR;
    const uint32_t lp = (uint32_t)(rr * ROWB + (((lane % CPR) ^ pf32_swz<D>(rr)) << 4));
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int k = (wave * IPW + j) % KVI;
      cp_v[j] = lp ^ ((uint32_t)(pf32_swz<D>(RPC * k) ^ pf32_swz<D>(0)) << 4);
    }
  }
  // The item's 16-key tiles in batches of 64 (32 steps): lane i holds tile i of the current batch,
  // its byte offset from the head's first block (block offset plus row offset) and whether its
  // block-table entry names a block of the pool (an entry outside it marks the tile absent: block 0
  // is read in its place and every key of the tile is masked, so none reaches a product). Tiles are
  // 16-aligned and block_size is a multiple of 16, so a tile never straddles two blocks. In the step
  // holding key L - 1 a second tile past it repeats that tile; keys at or past L are masked out of S
  // and zeroed in the V image. The entries of a batch are gathered one batch ahead by a copy into
  // this wave's LDS table (counted with the KV copies, so the step waits cover it).
  const int bs = a.block_size;
  const int last_bi = (int)div_invariant((uint32_t)last_tile, a.bs_magic, a.bs_shift);
  const uint32_t bbytes = (uint32_t)a.block_bytes;
  const int32_t* bt_row = a.block_tables + (int64_t)it.seq * a.max_blocks;
  uint32_t t_lo = 0, t_hi = 0, t_ok = 0;  // this lane's tile of the current batch
  uint32_t s_lo = 0, s_hi = 0;            // (per token-head scales) offset of its scale rows
  int r_next = 0;                         // row of this lane's tile of the gathered batch
  // (the lane index is recomputed in these two: kept across the step loop, values derived from it
  // would be spilled and their reloads would wait for the copies in flight)
  auto lane_now = [&]() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  auto gather = [&](int batch) {
    const int kt = min(k_begin + kTileKeys * (64 * batch + lane_now()), last_tile);
    const int bi = (int)div_invariant((uint32_t)kt, a.bs_magic, a.bs_shift);
    r_next = kt - bi * bs;
    dma4_to_lds(bt_row + min(bi, last_bi), (uint32_t)(TBL + ((batch & 1) * 4 + wave) * 256));
  };
  auto load_batch = [&](int batch) {
    const int32_t e = *(const int32_t*)(smem + TBL + ((batch & 1) * 4 + wave) * 256 + 4 * lane_now());
    const bool ok = (uint32_t)e < (uint32_t)a.num_blocks;
    const uint64_t pg = ok ? (uint64_t)(uint32_t)e * bbytes : 0ull;
    const uint64_t to = pg + (uint32_t)(r_next * ROWB);
    t_lo = (uint32_t)to;
    t_hi = (uint32_t)(to >> 32);
    t_ok = ok ? 1u : 0u;
    if constexpr (PTH) {
      const uint64_t so = pg + (uint32_t)(bs * D + 4 * r_next);
      s_lo = (uint32_t)so;
      s_hi = (uint32_t)(so >> 32);
    }
  };
  auto rl64 = [&](uint32_t lo, uint32_t hi, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, l) << 32) | (uint32_t)__builtin_amdgcn_readlane((int)lo, l);
  };
  int okr[NS] = {0, 0, 0, 0};  // present tiles of the step in each ring stage (bit 0: first, bit 1: second)
  const int64_t kv_gap = vbase - kbase;
  // A step's codes travel through registers: the wave loads its IPW 16-byte chunks per lane (the last
  // wave at per-token-head scales also 16 bytes of scales in lanes 0..15) two iterations before the
  // step's K codes are first read, and writes them into the step's ring stage at the end of the next
  // iteration. (The direct global -> LDS copy serialises a wave's copies; plain loads keep many in
  // flight.)
  struct Staged {
    uint4 c[IPW];
    uint4 sc;
  };
  auto load_step = [&](auto uc, int s) {
    constexpr int U = decltype(uc)::value;  // ring stage: s % NS
    Staged r;
    if ((s & 31) == 0 && s > 0) {
      // a new batch: its entries (gathered a batch ago) into the lanes, and the next batch's gather
      load_batch(s >> 5);
      if (s + 32 < n_steps) gather((s >> 5) + 1);
    }
    const int li = 2 * (s & 31);
    okr[U] = __builtin_amdgcn_readlane((int)t_ok, li) | (__builtin_amdgcn_readlane((int)t_ok, li + 1) << 1);
    // the wave's tiles: IPW / TPC groups of TPC chunks, one tile each, 1 KB apart
    static_for<IPW / TPC>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      const int ii0 = wave * IPW + g * TPC;
      const int tsel = (RPC * (ii0 % KVI)) >> 4;
      const uint8_t* tb = kbase + (ii0 >= KVI ? kv_gap : 0) + rl64(t_lo, t_hi, li + tsel);
#pragma unroll
      for (int j = 0; j < TPC; ++j) r.c[g * TPC + j] = *(const uint4*)(tb + cp_v[g * TPC + j] + 1024 * j);
    });
    if constexpr (PTH) {
      if (wave == WAVES - 1) {
        // 16 lanes x 16 bytes: [K scales of the 32 keys][V scales], 4 scales per lane
        const int tt = (lane >> 2) & 1, part = lane & 3, kv = lane >> 3;
        const uint64_t so0 = rl64(s_lo, s_hi, li), so1 = rl64(s_lo, s_hi, li + 1);
        const uint8_t* src = (kv ? vbase : kbase) + (tt ? so1 : so0) + 16 * part;
        r.sc = lane < 16 ? *(const uint4*)src : make_uint4(0, 0, 0, 0);
      }
    }
    return r;
  };
  const uint32_t st_off = (uint32_t)(wave * IPW * 1024 + 16 * lane);  // the wave's chunks in a stage
  auto store_step = [&](auto uc, Staged r) {
    constexpr int U = decltype(uc)::value;  // ring stage of the step
#pragma unroll
    for (int j = 0; j < IPW; ++j) *(uint4*)(smem + st_off + (RB + U * STAGE + 1024 * j)) = r.c[j];
    if constexpr (PTH) {
      if (wave == WAVES - 1 && lane < 16) {
        // the K scales (lanes 0 .. 7) are staged times the logit scale, one multiply per key here
        // instead of one per logit in every wave
        float4 sc = __builtin_bit_cast(float4, r.sc);
        if (lane < 8) { sc.x *= xscale; sc.y *= xscale; sc.z *= xscale; sc.w *= xscale; }
        *(float4*)(smem + RB + U * STAGE + 2 * KT * ROWB + 16 * lane) = sc;
      }
    }
  };

  // ---- per-lane LDS offsets, fixed for the kernel (the ring stage, V image and block of each
  // access are constants added in the instruction's offset field)
  // K operands of S^T = K Q^T: key r32's chunk c (depth hh * D/2 + 8 c .. + 7) is half of the 16-byte
  // read c / 2 of the key's row
  uint32_t k_off[QC / 2];
#pragma unroll
  for (int m = 0; m < QC / 2; ++m)
    k_off[m] = (uint32_t)(RB + r32 * ROWB + (((hh * (CPR / 2) + m) ^ pf32_swz<D>(r32)) << 4));
  // V image of one step: block (dt, kc) holds, for lane l, head-dim column 32 dt + l % 32 of the keys
  // 16 kc + 8 (j / 4) + 4 h + j % 4 (j = 0..7, h = l / 32). A 16-lane group reads them from the ring
  // with one transposed read: its lanes 2i, 2i+1 point at the two 8-byte halves of key row i's 16
  // columns.
  uint32_t tr_off[VB_PW];
  {
    const int g16 = lane >> 4;
    const int tr_i = (lane & 15) >> 1;
    const int tr_key = 8 * (tr_i >> 2) + 4 * (g16 >> 1) + (tr_i & 3);  // key within a 16-key chunk
#pragma unroll
    for (int j = 0; j < VB_PW; ++j) {
      const int blk = wave * VB_PW + j;
      const int dt = blk >> 1, kc = blk & 1;
      const int key = 16 * kc + tr_key;
      const int lc = 2 * dt + (g16 & 1);
      tr_off[j] = (uint32_t)(RB + KT * ROWB + key * ROWB + ((lc ^ pf32_swz<D>(key)) << 4) + 8 * (lane & 1));
    }
  }
  // K image of one step: block i (i = 0 .. QC - 1) holds, for consumer lane l, the codes of key l % 32
  // at depth (l / 32) D/2 + 8 i .. + 7 widened to bf16 (the S^T operand of chunk i, read as 64 lanes x
  // 16 bytes). Each lane widens KU consecutive units of one key row: group g = 2 wave + lane / 32
  // takes units g KU .. of the row's 2 QC (lane half kh = g KU / QC, first chunk ki = g KU % QC).
  uint32_t kr_off[(KU + 1) / 2];  // its ring reads: 16-byte chunks (one 8-byte half when KU == 1)
  uint32_t kw_off;                 // its image writes (block ki, then 1024 bytes per further unit)
  {
    const int u0 = (2 * wave + hh) * KU;
    const int kh = u0 / QC, ki = u0 % QC;
    const int dep = kh * (D / 2) + 8 * ki;  // the first code of the lane's units in the key row
#pragma unroll
    for (int c = 0; c < (KU + 1) / 2; ++c)
      kr_off[c] = (uint32_t)(RB + r32 * ROWB + ((((dep >> 4) + c) ^ pf32_swz<D>(r32)) << 4) + (dep & 15));
    kw_off = (uint32_t)(KIM + (r32 + 32 * kh) * 16 + 1024 * ki);
  }
  const uint32_t l16 = (uint32_t)(lane * 16);                                   // V and K image reads
  const uint32_t vw_off = (uint32_t)(wave * VB_PW * 1024 + lane * 16);          // V image writes
  const uint32_t scl_off = (uint32_t)(RB + 2 * KT * ROWB + 16 * hh);            // scales: 4 hh floats in
  auto lds = [&](uint32_t off) { return smem + off; };

  float m_run = -INFINITY, l_run = 0.0f;  // per lane: the row's reference max, its partial sum
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  // The V image of step `sm` from its codes (already read into trc): a tile that is absent, and
  // keys at or past L, become zeros (the work-group agrees on this, every wave reading the image).
  auto v_image = [&](auto vc, auto mc, const i32x2 (&trc)[VB_PW], int sm) {
    constexpr int VOI = decltype(vc)::value;
    constexpr bool MASK = decltype(mc)::value != 0;
    const int ok = okr[sm % NS];
    const int nv = it.L - (k_begin + sm * KT + 4 * hh);  // valid keys from this lane's first key
#pragma unroll
    for (int j = 0; j < VB_PW; ++j) {
      uint32_t c0 = (uint32_t)trc[j].x, c1 = (uint32_t)trc[j].y;
      if constexpr (MASK) {
        const int kc = (wave * VB_PW + j) & 1;
        const int n0 = nv - 16 * kc, n1 = n0 - 8;
        uint32_t m0 = n0 >= 4 ? 0xFFFFFFFFu : (n0 <= 0 ? 0u : (1u << (8 * n0)) - 1u);
        uint32_t m1 = n1 >= 4 ? 0xFFFFFFFFu : (n1 <= 0 ? 0u : (1u << (8 * n1)) - 1u);
        if (!((ok >> kc) & 1)) { m0 = 0u; m1 = 0u; }
        c0 &= m0;
        c1 &= m1;
      }
      *(bf16x8*)lds(vw_off + VOI + 1024 * j) = widen8<DT>(c0, c1);
    }
  };

  // The K image of the step in ring stage `kc` into image slot `kw`: codes read, then widened
  // and written (no masking: the logits of masked keys are replaced)
  auto k_codes = [&](auto kc, uint32_t (&kb)[2 * KU]) {
    constexpr int KBS = decltype(kc)::value * STAGE;
    if constexpr (KU == 1) {
      const uint2 v = *(const uint2*)lds(kr_off[0] + KBS);
      kb[0] = v.x;
      kb[1] = v.y;
    } else {
#pragma unroll
      for (int c = 0; c < KU / 2; ++c) {
        const uint4 v = *(const uint4*)lds(kr_off[c] + KBS);
        kb[4 * c] = v.x;
        kb[4 * c + 1] = v.y;
        kb[4 * c + 2] = v.z;
        kb[4 * c + 3] = v.w;
      }
    }
  };
  auto k_image = [&](auto kw, const uint32_t (&kb)[2 * KU]) {
    constexpr int KIW = decltype(kw)::value;
#pragma unroll
    for (int j = 0; j < KU; ++j) *(bf16x8*)lds(kw_off + KIW + 1024 * j) = widen8<DT>(kb[2 * j], kb[2 * j + 1]);
  };

  // ---- prologue helpers: S of one step as one dependent chain (from the ring's codes), the V
  // image of step 0 and its (masked) softmax
  auto qk = [&](auto uc) {
    constexpr int KST = decltype(uc)::value * STAGE;
    f32x16 sv = {};
#pragma unroll
    for (int m = 0; m < QC / 2; ++m) {
      const uint4 c = *(const uint4*)lds(k_off[m] + KST);
      sv = mfma32x32x16(widen8<DT>(c.x, c.y), qb[2 * m], sv);
      sv = mfma32x32x16(widen8<DT>(c.z, c.w), qb[2 * m + 1], sv);
    }
    return sv;
  };
  // masked softmax of step 0; returns whether the reference maximum moved
  auto softmax0 = [&](const f32x16& sv, bf16x8 (&pbo)[2], float* alpha) {
    const int ok = okr[0];
    const bool ok0 = ok & 1, ok1 = ok & 2;
    const int kb = k_begin;
    const float* scl = (const float*)lds(scl_off);  // [K scales][V scales] of stage 0
    // visible keys [lo, hi) of the row, narrowed by an absent tile (the first: keys below kb + 16 go;
    // the second: keys from kb + 16 go); one unsigned compare per key
    const int lo = ok0 ? lo_r : max(lo_r, kb + kTileKeys);
    const int hi = ok1 ? hi_r : min(hi_r, kb + kTileKeys);
    const uint32_t width = hi > lo ? (uint32_t)(hi - lo) : 0u;
    const int base = kb + 4 * hh - lo;
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x[e] = PTH ? sv[e] * scl[8 * (e >> 2) + (e & 3)] : sv[e] * xscale;  // (staged K scales carry xscale)
      if constexpr (CAP) x[e] = a.softcap * kLog2e * tanh_via_exp2(x[e] * a.inv_softcap);
      if constexpr (ALIBI) x[e] += slope2 * (float)(kb + 8 * (e >> 2) + 4 * hh + (e & 3) - pos);
      if (!((uint32_t)(base + 8 * (e >> 2) + (e & 3)) < width)) x[e] = -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[e]);
    auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx), __builtin_bit_cast(uint32_t, mx), false, false);
    mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    // lazy rescaling: the reference maximum moves only when some row's logits exceed it by 8
    const bool grow = __builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0;
    const float m_new = grow ? fmaxf(m_run, mx) : m_run;
    *alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.0f : m_new));
    m_run = m_new;
    const float m_use = m_run == -INFINITY ? 0.0f : m_run;
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float pe = fast_exp2(x[e] - m_use);
      psum += pe;
      // a masked key may have an unwritten scale slot: select, do not multiply, its zero
      if constexpr (PTH) pe = x[e] == -INFINITY ? 0.0f : pe * scl[KT + 8 * (e >> 2) + (e & 3)];
      pbo[e >> 3][e & 7] = (__bf16)pe;
    }
    if constexpr (!PTH) {
      // (the row sum of the probabilities as they enter the PV product, as in the other steps)
      psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) psum += (float)pbo[e >> 3][e & 7];
    }
    l_run = (grow ? l_run * *alpha : l_run) + psum;
    return grow;
  };

  // ---- one step of the pipeline at ring phase U (= step % NS), in NSL slices kept in order: each
  // slice issues one MFMA of S of step + 2 (K operand from its image) and one of the PV product of
  // step (operands read two slices ahead), and a share of the vector work: the softmax of step + 1
  // (whose S is `s_in`) into the probabilities `pb_out`, the V image of step + 1 and the K image of
  // step + 3.
  // FULL: no key of step + 1 is masked for this wave and both its tiles are present. Returns whether
  // the reference maximum moved (then *alpha is the factor for the output, applied by the caller
  // once these PV products are done).
  auto slices = [&](auto uc, bool full, const f32x16& s_in, const bf16x8 (&pb_in)[2], f32x16& s_out,
                    bf16x8 (&pb_out)[2], int sm, float* alpha) {
    constexpr int U = decltype(uc)::value;
    constexpr int KIR = KIM + (U & 1) * VIMG;    // K image of step + 2 (slot (step + 2) % 2)
    constexpr int KIW = ((U + 1) & 1) * VIMG;    // slot of step + 3's K image (relative to KIM)
    constexpr int VST = ((U + 1) % NS) * STAGE;  // ring stage of step + 1: its V codes and scales
    constexpr int PVI = (U & 1) * VIMG;          // V image of step
    constexpr int VOI = ((U + 1) & 1) * VIMG;    // V image of step + 1
    // per-tensor scales, no soft-cap and no bias: the logit scale folds into the exponent (a masked
    // key's -inf stays -inf through it, the scale being positive)
    constexpr bool PLAIN = !PTH && !CAP && !ALIBI;
    const int ok = okr[(U + 1) % NS];
    const bool ok0 = ok & 1, ok1 = ok & 2;
    const int kb = k_begin + sm * KT;
    bf16x8 ko[NSL], vo[NSL];
    uint32_t kcode[2 * KU];  // codes of this lane's units of step + 3's K image
    i32x2 trc[VB_PW];
    float x[16], p[16];
    float4 ks4[4], vs4[4];
    // operands are read two slices ahead of their MFMA
    constexpr int VPF = 2, KPF = 2;
    static_assert(NSL >= 4, "the slices hold the prefetched operands");
#pragma unroll
    for (int m = 0; m < KPF; ++m) ko[m] = *(const bf16x8*)lds(l16 + KIR + 1024 * m);
#pragma unroll
    for (int i = 0; i < VPF; ++i) vo[i] = *(const bf16x8*)lds(l16 + PVI + 1024 * i);
    k_codes(IC<(U + 3) % NS>{}, kcode);
    if constexpr (PTH) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ks4[g] = *(const float4*)lds(scl_off + VST + 32 * g);
        vs4[g] = *(const float4*)lds(scl_off + VST + 4 * KT + 32 * g);
      }
    }
#pragma unroll
    for (int j = 0; j < VB_PW; ++j) trc[j] = lds_read_tr8(lds(tr_off[j] + VST));
    float mx = 0.0f, m_use = 0.0f;
    bool grow = false;
    // per-token-head scales without soft-cap or bias: each logit is taken relative to the current
    // reference (one multiply-add instead of a multiply and a subtraction); only a step that moves
    // the reference shifts them once more
    constexpr bool REL = PTH && !CAP && !ALIBI;
    const float m_old = m_run == -INFINITY ? 0.0f : m_run;
    constexpr int EXP0 = NSL >= 4 ? 2 : 1, EXPN = NSL >= 4 ? NSL - 3 : 1;  // slices holding the exps
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      if (i + KPF < NSL) ko[i + KPF] = *(const bf16x8*)lds(l16 + KIR + 1024 * (i + KPF));
      if (i + VPF < NSL) vo[i + VPF] = *(const bf16x8*)lds(l16 + PVI + 1024 * (i + VPF));
      s_out = mfma32x32x16(ko[i], qb[i], i == 0 ? f32x16{} : s_out);
      acc[i / 2] = mfma32x32x16(vo[i], pb_in[i % 2], acc[i / 2]);
      if (i == 0) {
        // logits (log2 domain) of keys kb + 8 (e / 4) + 4 hh + e % 4; a plain per-tensor step keeps
        // S as it is and folds the scale into the exponent's multiply-add below
#pragma unroll
        for (int e = 0; e < 16; ++e)
          x[e] = PLAIN ? s_in[e]
                       : (REL ? __builtin_fmaf(s_in[e], ks4[e >> 2][e & 3], -m_old)
                              : (PTH ? s_in[e] * ks4[e >> 2][e & 3] : s_in[e] * xscale));
        if constexpr (CAP) {
#pragma unroll
          for (int e = 0; e < 16; ++e) x[e] = a.softcap * kLog2e * tanh_via_exp2(x[e] * a.inv_softcap);
        }
        if constexpr (ALIBI) {
          // + slope * (key - position), after the soft-cap
          const int base = kb + 4 * hh - pos;
#pragma unroll
          for (int e = 0; e < 16; ++e) x[e] += slope2 * (float)(base + 8 * (e >> 2) + (e & 3));
        }
        if (!full) {
          // visible keys [lo, hi) of the row, narrowed by an absent tile (the first: keys below
          // kb + 16 go; the second: keys from kb + 16 go); one unsigned compare per key
          const int lo = ok0 ? lo_r : max(lo_r, kb + kTileKeys);
          const int hi = ok1 ? hi_r : min(hi_r, kb + kTileKeys);
          const uint32_t width = hi > lo ? (uint32_t)(hi - lo) : 0u;
          const int base = kb + 4 * hh - lo;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (!((uint32_t)(base + 8 * (e >> 2) + (e & 3)) < width)) x[e] = -INFINITY;
        }
        // (three-input maxima: v_max3_f32)
        float m0 = fmaxf(fmaxf(x[0], x[1]), x[2]);
        float m1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
        float m2 = fmaxf(fmaxf(x[6], x[7]), x[8]);
        float m3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
        float m4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
        m0 = fmaxf(fmaxf(m0, m1), m2);
        m3 = fmaxf(fmaxf(m3, m4), x[15]);
        mx = fmaxf(m0, m3);
      }
      if (i == (NSL >= 2 ? 1 : 0)) {
        auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx), __builtin_bit_cast(uint32_t, mx), false, false);
        mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
        // lazy rescaling: the reference maximum moves only when some row's logits exceed it by 8
        if constexpr (PLAIN) mx *= xscale;  // the logit scale is positive: max(x * scale) = max(x) * scale
        if constexpr (REL) mx += m_old;     // (the logits were taken relative to m_old)
        grow = __builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0;
        const float m_new = grow ? fmaxf(m_run, mx) : m_run;
        *alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.0f : m_new));
        m_run = m_new;
        m_use = m_run == -INFINITY ? 0.0f : m_run;
        if constexpr (REL) {
          // (the reference stays where it was unless it moved: then the logits shift once)
          if (grow) {
            const float d = m_use - m_old;
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] -= d;
          }
        }
      }
      if (i >= EXP0 && i < EXP0 + EXPN) {
        // exps e with e * EXPN / 16 == i - EXP0: an even spread of the 16 over the slices
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (e * EXPN / 16 == i - EXP0)
            p[e] = fast_exp2(PLAIN ? __builtin_fmaf(x[e], xscale, -m_use) : (REL ? x[e] : x[e] - m_use));
      }
      if (i == NSL / 2) {
        if (full) v_image(IC<VOI>{}, IC<0>{}, trc, sm);
        else v_image(IC<VOI>{}, IC<1>{}, trc, sm);
      }
      if (i == NSL / 2 - 1) k_image(IC<KIW>{}, kcode);
      if (i == NSL - 1) {
        float psum;
        if constexpr (PTH) {
          psum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])) +
                 ((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15]));
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] *= vs4[e >> 2][e & 3];
          if (!full) {
            // a masked key may have an unwritten scale slot: its product is replaced by zero
#pragma unroll
            for (int e = 0; e < 16; ++e) p[e] = x[e] == -INFINITY ? 0.0f : p[e];
          }
        }
        // (pairs: one v_cvt_pk_bf16_f32 each)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x2 pr = {p[8 * kk + 2 * j], p[8 * kk + 2 * j + 1]};
            const bf16x2 b = __builtin_convertvector(pr, bf16x2);
            pb_out[kk][2 * j] = b[0];
            pb_out[kk][2 * j + 1] = b[1];
          }
        if constexpr (!PTH) {
          // the row sum of the probabilities as they enter the PV product (bf16), two at a time
          psum = 0.0f;
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x2 pr = {pb_out[kk][2 * j], pb_out[kk][2 * j + 1]};
              psum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, psum, false);
            }
        }
        l_run = (grow ? l_run * *alpha : l_run) + psum;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return grow;
  };

  // ---- software pipeline. Prologue: steps 0 .. 3 into their stages, S of steps 0 and 1, the
  // softmax of step 0, its V image and the K image of step 2. Iteration t (0 <= t < n - 1), after
  // one barrier: the loads of step t + 4 start; the slices run S of step t + 2 (beyond the last
  // step: unused), the PV product of step t, the softmax and the V image of step t + 1 (whose S came
  // from iteration t - 1) and the K image of step t + 3; then step t + 4 goes into the stage step t
  // left. The PV product of the last step follows the loop. Each image is written one iteration
  // before it is read and each ring stage is read while later ones fill, so one barrier per step
  // orders every writer and reader. The loop is unrolled over the four ring stages, so every LDS
  // offset is a constant and S, the probabilities and the images alternate between two buffers
  // without copies. A move of the reference maximum (rare) stops the loop after the iteration whose
  // PV product still used the old one; the output is rescaled outside the loop, so inside it only
  // matrix instructions touch the output and it stays in the matrix accumulation registers.
  if (n_steps > 0) {
    // the first batch's entries (waited for here, before any KV copy), then the second's gather
    gather(0);
    wait_vmcnt_c<0>();
    load_batch(0);
    if (n_steps > 32) gather(1);
  }
  {
    Staged t0, t1, t2, t3;
    if (n_steps > 0) t0 = load_step(IC<0>{}, 0);
    if (n_steps > 1) t1 = load_step(IC<1>{}, 1);
    if (n_steps > 2) t2 = load_step(IC<2>{}, 2);
    if (n_steps > 3) t3 = load_step(IC<3>{}, 3);
    load_q();
    if (n_steps > 0) store_step(IC<0>{}, t0);
    if (n_steps > 1) store_step(IC<1>{}, t1);
    if (n_steps > 2) store_step(IC<2>{}, t2);
    if (n_steps > 3) store_step(IC<3>{}, t3);
  }
  f32x16 sA, sB;     // S of the even and of the odd steps
  bf16x8 pA[2], pB[2];  // probabilities of the even and of the odd steps
  if (n_steps > 0) {
    __syncthreads();  // stages 0 .. 3 written by every wave
    // S of steps 0 and 1 (from the codes), the V image of step 0, the K image of step 2 and the
    // softmax of step 0 (the output is still zero: a move of the reference maximum needs no rescale)
    const f32x16 s0 = qk(IC<0>{});
    if (n_steps > 1) sB = qk(IC<1>{});
    {
      i32x2 trc[VB_PW];
#pragma unroll
      for (int j = 0; j < VB_PW; ++j) trc[j] = lds_read_tr8(lds(tr_off[j]));
      v_image(IC<0>{}, IC<1>{}, trc, 0);
      uint32_t kb[2 * KU];
      k_codes(IC<2>{}, kb);
      k_image(IC<0>{}, kb);
    }
    float alpha0;
    softmax0(s0, pA, &alpha0);
  }
  int step = 0;
  float alpha = 1.0f;
  bool rescale = false;
  // one iteration at ring phase U = step % NS; true when the loop stops (no next step, or a move of
  // the reference maximum: then `rescale`)
  auto iter = [&](auto uc) {
    constexpr int U = decltype(uc)::value;
    if (step + 1 >= n_steps) return true;
    __syncthreads();  // stage step + 3, the V image of step and the K image of step + 2 written by every wave
    Staged st;
    if (step + 4 < n_steps) st = load_step(IC<U>{}, step + 4);
    const int s1 = step + 1;
    const bool full = s1 >= f_lo && s1 <= f_hi && okr[(U + 1) % NS] == 3;
    f32x16& s_in = pick<(U + 1) & 1>(sA, sB);
    f32x16& s_out = pick<U & 1>(sA, sB);
    bf16x8(&pb_in)[2] = pick<U & 1>(pA, pB);
    bf16x8(&pb_out)[2] = pick<(U + 1) & 1>(pA, pB);
    rescale = slices(uc, full, s_in, pb_in, s_out, pb_out, s1, &alpha);
    // step + 4 into the stage step left (read from the next iteration on: its barrier orders the
    // writes)
    if (step + 4 < n_steps) store_step(IC<U>{}, st);
    step = s1;
    return rescale;
  };
  for (;;) {
    // every vector memory access the compiler placed before the loop (spill reloads after a rescale)
    // completes here, rarely, so it places no wait for them inside the loop, where such a wait would
    // also drain the copies in flight (s_waitcnt vmcnt(0): gfx9 encoding, the other counters free)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    rescale = false;
    // (one entry, at the top: after a rescale the phases before the current one are skipped once)
    for (;;) {
      if ((step & 3) == 0 && iter(IC<0>{})) break;
      if ((step & 3) == 1 && iter(IC<1>{})) break;
      if ((step & 3) == 2 && iter(IC<2>{})) break;
      if ((step & 3) == 3 && iter(IC<3>{})) break;
    }
    if (!rescale) break;
    // (one head-dim tile at a time, so few registers hold a copy of the output)
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      acc[t] *= alpha;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (n_steps > 0) {
    // the PV product of the last step (its V image was written by every wave)
    wait_vmcnt_c<0>();
    __syncthreads();
    auto pv = [&](auto pc, const bf16x8 (&pbi)[2]) {
      constexpr int PVI = decltype(pc)::value;
#pragma unroll
      for (int i = 0; i < NSL; ++i) acc[i / 2] = mfma32x32x16(*(const bf16x8*)lds(l16 + PVI + 1024 * i), pbi[i % 2], acc[i / 2]);
    };
    if ((n_steps - 1) & 1) pv(IC<VIMG>{}, pB);
    else pv(IC<0>{}, pA);
  }
  // ---- normalise and write the row (a run of a split item: its partial result instead). The
  // lane's accumulator i holds head-dim element 32 dt + 8 (i / 4) + 4 hh + i % 4.
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, l_run), __builtin_bit_cast(uint32_t, l_run), false, false);
    l_run = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
  }
  if (!row_ok) return;
  if (it.slot >= 0) {
    const int64_t sl = (int64_t)it.slot + row;
    float* pp = a.scratch + sl * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(pp + 32 * dt + 8 * g + 4 * hh) =
            make_float4(acc[dt][4 * g] * a.v_scale, acc[dt][4 * g + 1] * a.v_scale, acc[dt][4 * g + 2] * a.v_scale,
                        acc[dt][4 * g + 3] * a.v_scale);
    if (hh == 0) {
      float* ml = a.scratch + a.num_slots * D + sl * 2;
      ml[0] = m_run;
      ml[1] = l_run;
    }
    return;
  }
  float f = 1.0f, lt = l_run;
  if (a.sinks) {
    // the sink logit joins the normaliser: rescale to the larger of it and the row's reference
    const float M = fmaxf(m_run, sink2);
    f = fast_exp2(m_run - M);
    lt = lt * f + fast_exp2(sink2 - M);
  }
  // a row with no key left (every block of its range outside the pool) and no sink writes 0
  const float norm = lt > 0.0f ? a.v_scale * f / lt : 0.0f;
  uint16_t* op = a.out + orow;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16_rne(acc[dt][4 * g] * norm) | ((uint32_t)f32_to_bf16_rne(acc[dt][4 * g + 1] * norm) << 16);
      w.y = (uint32_t)f32_to_bf16_rne(acc[dt][4 * g + 2] * norm) | ((uint32_t)f32_to_bf16_rne(acc[dt][4 * g + 3] * norm) << 16);
      *(uint2*)(op + 32 * dt + 8 * g + 4 * hh) = w;
    }
}

template <int D, int DT, int MODE, int WAVES>
static int launch_pf32_w(const AttnArgs& a, hipStream_t st) {
  const SchedHeader& h = *a.hdr;
  Pf32Args p;
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
  const dim3 grid(h.num_pf_items), block(WAVES * 64);
  const bool cap = a.softcap > 0.0f, alibi = a.alibi_slopes != nullptr;
  if (cap && alibi)
    hipLaunchKernelGGL((prefill32_kernel<D, DT, MODE, true, true, WAVES>), grid, block, h.pf_lds_bytes, st, p);
  else if (cap)
    hipLaunchKernelGGL((prefill32_kernel<D, DT, MODE, true, false, WAVES>), grid, block, h.pf_lds_bytes, st, p);
  else if (alibi)
    hipLaunchKernelGGL((prefill32_kernel<D, DT, MODE, false, true, WAVES>), grid, block, h.pf_lds_bytes, st, p);
  else
    hipLaunchKernelGGL((prefill32_kernel<D, DT, MODE, false, false, WAVES>), grid, block, h.pf_lds_bytes, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("aqp_paged_attention: prefill launch failed: %s", hipGetErrorString(e));
    return AQP_ERR_HIP;
  }
  return AQP_OK;
}

template <int D, int DT, int MODE>
static int launch_pf32(const AttnArgs& a, hipStream_t st) {
  const int rows = a.hdr->pf_rows;
  if (rows == kPfRows) return launch_pf32_w<D, DT, MODE, kPfRows / 32>(a, st);
  if (rows == kPfRowsSmall) return launch_pf32_w<D, DT, MODE, kPfRowsSmall / 32>(a, st);
  set_error("aqp_paged_attention: schedule rows per prefill item %d not built", rows);
  return AQP_ERR_SCHEDULE_MISMATCH;
}

template <int DT, int MODE>
static int pf32_d(const AttnArgs& a, hipStream_t st) {
  switch (a.head_dim) {
    case 64: return launch_pf32<64, DT, MODE>(a, st);
    case 128: return launch_pf32<128, DT, MODE>(a, st);
  }
  set_error("aqp_paged_attention: unsupported head_dim %d", a.head_dim);
  return AQP_ERR_UNSUPPORTED;
}

int launch_prefill32(int dtype, int mode, const AttnArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E4M3) return pf32_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_FP8_E5M2) return pf32_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TENSOR && dtype == AQP_KV_INT8) return pf32_d<AQP_KV_INT8, AQP_SCALE_PER_TENSOR>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_INT8) return pf32_d<AQP_KV_INT8, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E4M3) return pf32_d<AQP_KV_FP8_E4M3, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  if (mode == AQP_SCALE_PER_TOKEN_HEAD && dtype == AQP_KV_FP8_E5M2) return pf32_d<AQP_KV_FP8_E5M2, AQP_SCALE_PER_TOKEN_HEAD>(a, st);
  set_error("aqp_paged_attention: dtype %d with scale mode %d has no 32x32 prefill", dtype, mode);
  return AQP_ERR_UNSUPPORTED;
}

}  // namespace aqp
