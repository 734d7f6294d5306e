// Library-internal definitions shared by the host code and the HIP kernels:
// cache geometry, schedule metadata layout and kernel launch entry points.
//
// The schedule records the element sizes and tile geometry it was built
// with; the launcher compares them with what the compiled kernels use and
// refuses a mismatch. This is the lesson of the "Fix CPU FP8 attention
// scheduler scratch sizing" page (vllm PR 50194, Motivation and Review):
// the scheduler sized tiles and scratch from one element size while the
// runtime used another, and a large prefill wrote past its scratch buffer.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/aqp.h"

namespace aqp {

constexpr uint32_t kMagic = 0x53505141u;  // "AQPS"
constexpr uint32_t kVersion = 4;

// ---- compile-time tile geometry of the kernels ----------------------------
constexpr int kTileKeys = 16;        // keys per KV tile: one 16-row MFMA operand
constexpr int kMaxBlockSize = 65536; // largest block size (keys per block)
constexpr int kDecIterKeys = 16;     // keys per decode iteration (one tile; PV on 16x16x16 MFMA)
constexpr int kDecWaves = 4;         // compute waves per decode work-group (they split a segment's iterations)
// q heads per decode unit (MFMA column block): 16, or at head_dim 256 8 (one-byte codes) or 4 (the
// unquantised cache, whose tiles take twice the ring) so the work-group's LDS (Q rows and the
// merge area grow with the heads) stays within one CU's
constexpr int heads_per_unit(int head_dim, int eb) { return head_dim >= 256 ? (eb == 2 ? 4 : 8) : 16; }
constexpr int kPfRows = 128;         // prefill: query rows (token, q head) per work item
// prefill: rows per item when 128-row items would leave CUs with fewer than two work-groups
// (head_dim <= 128): twice the items, so a CU overlaps one work-group's waits with another's work
constexpr int kPfRowsSmall = 64;
// Prefill waves per work-group: head_dim 256 gives each of 8 waves 16 rows (so a wave's
// 16 x 256 fp32 output tile and its Q rows stay in ordinary registers at two waves per SIMD);
// smaller head dims give each of 4 waves 32 rows, which halves the LDS operand reads per MFMA.
constexpr int pf_waves(int head_dim) { return head_dim >= 256 ? 8 : 4; }
constexpr int kPfKvTile = 32;        // prefill: keys staged in LDS per step
constexpr int kPfStages = 4;         // prefill: LDS ring stages of codes (two steps ahead of the widening)
// Ring stages of the 16x16 prefill: kPfStages, or three (one step ahead of the widening) where a
// stage holds 512-byte rows (the unquantised cache at head_dim 256), so that the ring and the
// operand images fill one CU's LDS exactly
constexpr int pf_stages(int head_dim, int eb) { return head_dim * eb >= 512 ? 3 : kPfStages; }
constexpr int kPfOperandBytes = 2;   // prefill: bf16 operand images in LDS
constexpr int kMinRunTiles = 32;     // decode: fewest 16-key tiles a work-group is given
// prefill key splits: when a batch has fewer prefill items than the device holds work-groups at
// once, long items are cut into runs of at least this many kPfKvTile-key steps (at most
// kPfMaxSplit runs each); the runs' partial results are merged like split decode ranges
constexpr int kPfMinSplitSteps = 16;
constexpr int kPfMaxSplit = 8;
constexpr int kCwRowsPerLane = 4;    // cache write: rows each lane loads before converting
constexpr int kCwWgsPerCu = 16;      // cache write: resident work-groups per CU (grid cap)
constexpr int kLdsPerCu = 160 * 1024;  // LDS bytes per compute unit (gfx950)
// Accelerator dies (XCDs) of the chip, each with its own L2: work-group i of a launch runs on XCD
// i % kXcds.
constexpr int kXcds = 8;
// Prefill work-groups a CU holds at once: the register limit of the compiled kernel (8 waves at two
// per SIMD at head_dim 256; 4 waves at two per SIMD at 128 rows and head_dim 128, three below)
// and the LDS limit. (Per-group scales at head_dim 64 spill some registers at three waves per
// SIMD, yet measured faster there than without the spill at two: 40.6 against 45.8 us on 8 x 512
// tokens, 32/8 heads.)
constexpr int pf_wgs_per_cu(int head_dim, int rows, int32_t lds_bytes) {
  return (head_dim >= 256 ? 1 : (head_dim == 128 && rows > kPfRowsSmall ? 2 : 3)) < kLdsPerCu / lds_bytes
             ? (head_dim >= 256 ? 1 : (head_dim == 128 && rows > kPfRowsSmall ? 2 : 3))
             : kLdsPerCu / lds_bytes;
}
// The 32x32 prefill kernel (prefill32.hip) serves one-byte codes with per-tensor or per-token-head
// scales up to head_dim 128, where it runs two waves per SIMD; per-group scales, the unquantised
// cache and head_dim 256 keep the 16x16 kernel (prefill.hip), which was measured faster there
// (a single wave per SIMD hides little of its vector work under its matrix instructions).
// Block sizes that are not a multiple of 16 (a 16-key tile may span several blocks) also keep the
// 16x16 kernel, which gathers such tiles row by row.
constexpr bool pf32_applies(int dtype, int mode, int head_dim, int block_size) {
  return head_dim <= 128 && dtype != AQP_KV_AUTO && (mode == AQP_SCALE_PER_TENSOR || mode == AQP_SCALE_PER_TOKEN_HEAD) &&
         block_size % kTileKeys == 0;
}
constexpr int kPf32Stages = 4;  // LDS ring stages of the 32x32 prefill (four steps ahead)
// Waves per SIMD its registers are sized for: a wave holds 32 rows of Q (D/4 registers), their
// fp32 output (D/2), the next step's K operands (D/4) and two S tiles. At head_dim 64 three waves
// (168 registers each) fit the per-tensor kernel; the per-token-head kernel (scales beside the
// logits and probabilities) would spill to scratch memory there, and takes two (measured: int8 per
// token-head 55 -> 37-45 us on 8 x 512 tokens, 32/8 heads).
constexpr int pf32_waves_per_simd(int head_dim, int mode) {
  return head_dim >= 256 ? 1 : (head_dim == 128 || mode == AQP_SCALE_PER_TOKEN_HEAD ? 2 : 3);
}
// Ring stage: the codes of kPfKvTile keys of K and of V, then (per token-head) their fp32 scales.
constexpr int pf32_stage_bytes(int head_dim, int mode) {
  return 2 * kPfKvTile * head_dim + (mode == AQP_SCALE_PER_TOKEN_HEAD ? 2 * kPfKvTile * 4 : 0);
}
// LDS of one 32x32 prefill work-group: two slots each holding a step's V image and two holding a
// step's K image (bf16, kPfKvTile x head_dim each), the ring, then the block-table entries of two
// batches of 64 tiles for each of up to 4 waves (4 bytes each).
constexpr int kPf32TableBytes = 2 * 4 * 64 * 4;
constexpr int32_t pf32_lds_bytes(int head_dim, int mode) {
  return kPf32Stages * pf32_stage_bytes(head_dim, mode) + 4 * kPfKvTile * head_dim * 2 + kPf32TableBytes;
}
constexpr int pf32_wgs_per_cu(int head_dim, int mode, int rows, int32_t lds_bytes) {
  return 4 * pf32_waves_per_simd(head_dim, mode) / (rows / 32) < kLdsPerCu / lds_bytes
             ? 4 * pf32_waves_per_simd(head_dim, mode) / (rows / 32)
             : kLdsPerCu / lds_bytes;
}
// fp32 scales stored per cache row: none per tensor, one per token-head, head_dim / 32 per group
constexpr int row_scales(int head_dim, int mode) {
  return mode == AQP_SCALE_PER_TOKEN_HEAD ? 1 : (mode == AQP_SCALE_PER_GROUP ? head_dim / AQP_SCALE_GROUP : 0);
}
// prefill: scale bytes of one ring stage (K and V of kPfKvTile keys; at least one float per key
// for the codes, none for the unquantised cache)
constexpr int pf_stage_scale_bytes(int head_dim, int mode, int eb) {
  return eb == 2 ? 0 : 2 * kPfKvTile * 4 * (row_scales(head_dim, mode) > 1 ? row_scales(head_dim, mode) : 1);
}
// prefill: scale bytes after each of the two V images (a step's K and V scales; none for the
// unquantised cache)
constexpr int pf_vslot_scale_bytes(int eb) { return eb == 2 ? 0 : 2 * kPfKvTile * 4; }

// Decode LDS: per compute wave, a ring of dec_stages tiles (each the K and V codes of 16 keys plus
// their per-token-head scales) and one Q slot (the q rows of one segment); then the merge area
// where the compute waves hand their (O, m, l) to the merging wave.
// (eb: bytes per stored element, 1 for the codes, 2 for the unquantised bf16 cache)
constexpr int dec_stages(int head_dim, int eb) { return head_dim * eb >= 256 ? 2 : 3; }
constexpr int dec_slot_bytes(int head_dim, int mode, int eb) {
  return 2 * kDecIterKeys * head_dim * eb + 2 * kDecIterKeys * 4 * row_scales(head_dim, mode);
}
// Floats per (wave, head) row of the merge area: D of O, then m and l, padded to a multiple of 4
// so each lane's 4 consecutive values move as one 16-byte LDS access; with D/4 + 1 16-byte units
// per row, the 16 heads of a 16-lane pass start on 16 distinct units (no bank conflicts).
constexpr int merge_stride(int head_dim) { return head_dim + 4; }
constexpr int32_t dec_lds_bytes(int head_dim, int mode, int group_heads, int eb) {
  return kDecWaves * (dec_stages(head_dim, eb) * dec_slot_bytes(head_dim, mode, eb) + group_heads * head_dim * 2) +
         kDecWaves * group_heads * merge_stride(head_dim) * 4;
}
// Waves per SIMD the decode kernel's registers are sized for; a work-group is kDecWaves compute
// waves and one merging wave.
constexpr int dec_waves_per_simd(int head_dim) { return head_dim <= 128 ? 3 : 2; }
// Decode work-groups resident per CU: the smaller of the register limit of the compiled kernel
// and the LDS limit. The decode grid is exactly one resident wave of work-groups.
constexpr int decode_wgs_per_cu(int head_dim, int32_t lds_bytes) {
  return 4 * dec_waves_per_simd(head_dim) / (kDecWaves + 1) < kLdsPerCu / lds_bytes
             ? 4 * dec_waves_per_simd(head_dim) / (kDecWaves + 1)
             : kLdsPerCu / lds_bytes;
}
// Unsigned division by a divisor d >= 2 fixed for a launch, exact for every 32-bit n (division
// by an invariant integer with a multiply-high, the "round-up" method of Granlund and Montgomery):
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1; n / d = (t + ((n - t) >> 1)) >> (l - 1) with
// t = mulhi(n, m). The host computes (m, l - 1); the kernels apply it (div_invariant).
inline void invariant_divisor(uint32_t d, uint32_t* m, int32_t* shift) {
  if (d < 2) {  // not covered by the method: callers divide by 1 themselves
    *m = 0;
    *shift = 0;
    return;
  }
  int l = 0;
  while ((1ull << l) < d) ++l;
  *m = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
  *shift = l - 1;
}

// Compute units of the current device (256 on MI355X; 256 when no device is visible).
int device_cu_count();

// Geometry derived from the cache descriptor. One function computes it for
// both the scheduler and the launcher.
struct Geometry {
  int32_t head_dim;
  int32_t block_size;
  int32_t kv_elem_bytes;      // bytes per stored K/V element (1 for every supported dtype)
  int32_t staged_elem_bytes;  // bytes per element as staged in LDS by the kernels
  int32_t scale_bytes;        // inline scale bytes per row (4 per token-head, else 0)
  int32_t pad_;
  int64_t page_bytes;
  int64_t block_bytes;
  int64_t total_bytes;
  int32_t pf_lds_bytes;       // LDS per prefill work-group
};

// Fills g; returns AQP_OK or an error status with *why set.
int make_geometry(const aqp_cache_desc& d, Geometry* g, const char** why);

// ---- schedule metadata -----------------------------------------------------
// Layout: [SchedHeader][DecSeg x num_dec_segs][int32 dec_wg_start x (num_dec_wgs + 1)]
//         [DecSeg x num_dec_wgs: first segment of each work-group][CombItem x num_comb]
//         [PfItem x num_pf_items][int32 seq_lens x num_seqs], each array 256-byte aligned.
struct SchedHeader {
  uint32_t magic, version;
  // what the schedule was built for
  int32_t dtype, mode, kv_elem_bytes, staged_elem_bytes, scale_bytes;
  int32_t head_dim, block_size, num_blocks, num_q_heads, num_kv_heads;
  int32_t causal, window, max_blocks_per_seq, num_seqs;
  float sm_scale, softcap;
  int32_t total_q_tokens;
  // tile geometry the work items were cut with
  int32_t tile_keys, dec_iter_keys, dec_waves, pf_rows, pf_kv_tile, heads_per_unit;
  int32_t dec_lds_bytes, pf_lds_bytes;
  // work
  int32_t num_dec_wgs, num_dec_segs, num_parts, num_comb, num_pf_items, group_heads;
  int64_t off_dec_segs, off_dec_wg_start, off_comb, off_pf_items;
  int64_t meta_bytes, scratch_bytes;
  int64_t page_bytes, block_bytes;
  int64_t dec_kv_keys;  // total visible (key, KV head) pairs of the decode work (for reporting)
  int64_t off_seq_lens;  // keys of each sequence (the decode query of sequence b sits at seq_lens[b] - 1)
  // partial-result slots of the scratch: decode parts (num_parts x group_heads rows), then the
  // rows of split prefill runs; O of slot s at float s * head_dim, (m, l) at num_slots * head_dim + 2 s
  int64_t num_slots;
  int64_t comb_heads;    // most heads of one merge item (the merge grid's second dimension)
  int64_t num_pf_split;  // prefill runs that write partial results
  int64_t num_dec_comb;  // merge items [0, num_dec_comb) merge decode parts, the rest prefill runs
  int64_t off_dec_first; // DecSeg x num_dec_wgs: each work-group's first segment (zeros if it has none)
};

static_assert(offsetof(SchedHeader, off_dec_segs) == 136, "SchedHeader layout is part of the metadata format");
static_assert(sizeof(SchedHeader) == 256, "SchedHeader layout is part of the metadata format");

// Decode segment: keys [k_lo, k_hi) of (sequence, KV head, q heads
// [head0, head0 + nheads) of that KV head's group), one query token.
// part < 0: the segment is the whole visible range -> write the output;
// otherwise write partial (m, l, O) slot `part` of the scratch.
struct DecSeg {
  int32_t seq, kvh, head0, nheads, k_lo, k_hi, q_tok, part;
};

// Merge of num_parts partial results into the output rows of q heads [head0, head0 + nheads)
// of KV head kvh, query token q_tok: part s of head h is slot first_slot + s * part_stride + h
// (a split decode unit: its parts' slots; a split prefill run: the token's row in each run).
struct CombItem {
  int32_t kvh, head0, nheads, q_tok, first_slot, num_parts, part_stride, pad0;
};

// Prefill item: query tokens [q_lo, q_hi) (indices within the sequence) of
// sequence seq, all G q heads of KV head kvh. The sequence has L keys and ql
// queries; its first query is token q_start of q / out.
// Prefill item: query tokens [q_lo, q_hi) of sequence seq times q heads [head0, head0 + nheads)
// of KV head kvh; row r is token q_lo + r / nheads, head head0 + r % nheads.
// Keys outside [split_lo, split_hi) are not this item's (a run of a split item); slot >= 0: the
// item writes row r's partial result (O, m, l) to slot `slot + r` instead of the output.
struct PfItem {
  int32_t seq, kvh, q_lo, q_hi, L, ql, q_start, k_hi_max, head0, nheads, causal, split_lo;
  int32_t split_hi, slot, pad0, pad1;
};

// Scratch of one partial-result slot (one query row): D floats of O, then m and l.
inline int64_t slot_floats(int32_t head_dim) { return (int64_t)head_dim + 2; }

// ---- kernel launchers (defined in the .hip files) ---------------------------
struct CacheWriteArgs {
  uint8_t* cache;
  const uint16_t* k;
  const uint16_t* v;
  const int64_t* slots;
  int64_t num_tokens, token_stride;
  int64_t page_bytes, block_bytes;
  int64_t total_slots;
  int32_t num_kv_heads, head_dim, block_size;
  float k_scale, v_scale;
  int32_t narrow;  // rows (2 x tokens x KV heads) and slots below 2^31: 32-bit index arithmetic
  // n / num_kv_heads and n / block_size for 32-bit n by multiply-high (set when narrow; the head
  // count may be 1, which the method does not cover: then narrow is 0)
  uint32_t heads_magic, bs_magic;
  int32_t heads_shift, bs_shift;
};
int launch_cache_write(int dtype, int mode, const CacheWriteArgs& a, void* stream);

struct AttnArgs {
  const uint8_t* cache;
  const uint16_t* q;
  const int32_t* block_tables;
  const uint8_t* meta_dev;
  float* scratch;
  uint16_t* out;
  int64_t page_bytes, block_bytes;
  int32_t head_dim, block_size, num_kv_heads, num_q_heads, group, max_blocks_per_seq;
  int32_t window, causal;
  float sm_scale, softcap, k_scale, v_scale;
  const float* alibi_slopes;  // device [num_q_heads] or null
  const float* sinks;         // device [num_q_heads] or null
  const SchedHeader* hdr;  // host copy
};
int launch_decode(int dtype, int mode, const AttnArgs& a, void* stream);
// merges items [first, first + count) of the schedule's merge items (one wave per (item, head))
int launch_combine(const AttnArgs& a, int32_t first, int32_t count, void* stream);
int launch_prefill(int dtype, int mode, const AttnArgs& a, void* stream);
int launch_prefill32(int dtype, int mode, const AttnArgs& a, void* stream);

void set_error(const char* fmt, ...);

}  // namespace aqp
