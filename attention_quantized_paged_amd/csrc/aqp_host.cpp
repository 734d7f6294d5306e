// Host side of the C ABI: argument validation, cache geometry, the per-batch
// schedule, and kernel launches. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "aqp_internal.h"

namespace aqp {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

static int fail(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Which (dtype, mode) pairs are built: per-tensor fp8 (e4m3, e5m2) as on the
// PR 39445 page, per-token-head int8 / fp8 e4m3 as on the PR 38378 page, the
// two remaining code pairs, and the unquantised bf16 cache ("auto", no scales).
static int check_dtype_mode(int32_t dtype, int32_t mode, const char** why) {
  if (mode != AQP_SCALE_PER_TENSOR && mode != AQP_SCALE_PER_TOKEN_HEAD && mode != AQP_SCALE_PER_GROUP) { *why = "unknown scale mode"; return AQP_ERR_INVALID; }
  if (dtype == AQP_KV_AUTO && mode != AQP_SCALE_PER_TENSOR) { *why = "an unquantised cache has no stored scales"; return AQP_ERR_UNSUPPORTED; }
  if (dtype != AQP_KV_AUTO && dtype != AQP_KV_FP8_E4M3 && dtype != AQP_KV_FP8_E5M2 && dtype != AQP_KV_INT8) { *why = "unknown kv dtype"; return AQP_ERR_INVALID; }
  return AQP_OK;
}

int make_geometry(const aqp_cache_desc& d, Geometry* g, const char** why) {
  int rc = check_dtype_mode(d.dtype, d.mode, why);
  if (rc) return rc;
  if (d.num_blocks < 0 || d.num_kv_heads <= 0 || d.block_size <= 0 || d.head_dim <= 0) { *why = "non-positive cache dimension"; return AQP_ERR_INVALID; }
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256) { *why = "head_dim must be 64, 128 or 256"; return AQP_ERR_UNSUPPORTED; }
  // (any block size: the kernels gather a 16-key tile that spans several blocks row by row; the
  // bound keeps the float quotient of that gather exact)
  if (d.block_size > kMaxBlockSize || (int64_t)d.block_size * d.head_dim > (1ll << 30)) { *why = "block_size too large"; return AQP_ERR_UNSUPPORTED; }
  g->head_dim = d.head_dim;
  g->block_size = d.block_size;
  // bytes of one stored element: one per code; two for the unquantised bf16 cache. The kernels
  // stage raw elements in LDS, so the staged element has the same size.
  g->kv_elem_bytes = d.dtype == AQP_KV_AUTO ? 2 : 1;
  g->staged_elem_bytes = g->kv_elem_bytes;
  g->scale_bytes = 4 * row_scales(d.head_dim, d.mode);
  g->pad_ = 0;
  g->page_bytes = round_up((int64_t)d.block_size * d.head_dim * g->kv_elem_bytes + (int64_t)d.block_size * g->scale_bytes, 128);
  g->block_bytes = 2 * (int64_t)d.num_kv_heads * g->page_bytes;
  g->total_bytes = (int64_t)d.num_blocks * g->block_bytes;
  // Prefill work-group. The 32x32 kernel: a ring of kPf32Stages steps of codes (and scales) and
  // two V images of a step in bf16. The 16x16 kernel (per-group scales, head_dim 256, the
  // unquantised cache): a ring of pf_stages steps, each the K and V elements of kPfKvTile keys
  // plus their row scales; then two K and two V operand images of a step in bf16 (widened once
  // per work-group), each V image followed by a copy of its step's scales (none unquantised).
  if (pf32_applies(d.dtype, d.mode, d.head_dim, d.block_size))
    g->pf_lds_bytes = pf32_lds_bytes(d.head_dim, d.mode);
  else
    g->pf_lds_bytes = pf_stages(d.head_dim, g->staged_elem_bytes) *
                          (2 * kPfKvTile * d.head_dim * g->staged_elem_bytes +
                           pf_stage_scale_bytes(d.head_dim, d.mode, g->staged_elem_bytes)) +
                      4 * kPfKvTile * d.head_dim * kPfOperandBytes + 2 * pf_vslot_scale_bytes(g->staged_elem_bytes);
  return AQP_OK;
}

int device_cu_count() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cached = n;
    else
      cached = 256;
    (void)hipGetLastError();
  }
  return cached;
}

}  // namespace aqp

using namespace aqp;

extern "C" const char* aqp_last_error(void) { return g_last_error.c_str(); }

extern "C" int aqp_parse_kv_dtype(const char* s, int32_t* dtype, int32_t* mode) {
  if (!s || !dtype || !mode) return fail(AQP_ERR_INVALID, "aqp_parse_kv_dtype: null argument");
  struct { const char* name; int32_t dt, md; } table[] = {
      {"fp8", AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR},
      {"fp8_e4m3", AQP_KV_FP8_E4M3, AQP_SCALE_PER_TENSOR},
      {"fp8_e5m2", AQP_KV_FP8_E5M2, AQP_SCALE_PER_TENSOR},
      {"int8_per_token_head", AQP_KV_INT8, AQP_SCALE_PER_TOKEN_HEAD},
      {"fp8_per_token_head", AQP_KV_FP8_E4M3, AQP_SCALE_PER_TOKEN_HEAD},
      // the remaining codec x scale-mode pairs, named after the ones above
      {"int8", AQP_KV_INT8, AQP_SCALE_PER_TENSOR},
      {"fp8_e5m2_per_token_head", AQP_KV_FP8_E5M2, AQP_SCALE_PER_TOKEN_HEAD},
      // per-group scales (one per 32 head-dim channels), named the same way
      {"int8_per_group", AQP_KV_INT8, AQP_SCALE_PER_GROUP},
      {"fp8_per_group", AQP_KV_FP8_E4M3, AQP_SCALE_PER_GROUP},
      {"fp8_e5m2_per_group", AQP_KV_FP8_E5M2, AQP_SCALE_PER_GROUP},
  };
  for (auto& e : table) {
    if (std::strcmp(s, e.name) == 0) { *dtype = e.dt; *mode = e.md; return AQP_OK; }
  }
  if (std::strcmp(s, "auto") == 0) {  // the unquantised cache: bf16 elements, no scales
    *dtype = AQP_KV_AUTO;
    *mode = AQP_SCALE_PER_TENSOR;
    return AQP_OK;
  }
  return fail(AQP_ERR_INVALID, "unknown kv_cache_dtype '%s'", s);
}

extern "C" int aqp_cache_bytes(const aqp_cache_desc* desc, size_t* page_bytes, size_t* block_bytes, size_t* total_bytes) {
  if (!desc) return fail(AQP_ERR_INVALID, "aqp_cache_bytes: null descriptor");
  Geometry g;
  const char* why = "";
  int rc = make_geometry(*desc, &g, &why);
  if (rc) return fail(rc, "aqp_cache_bytes: %s", why);
  if (page_bytes) *page_bytes = (size_t)g.page_bytes;
  if (block_bytes) *block_bytes = (size_t)g.block_bytes;
  if (total_bytes) *total_bytes = (size_t)g.total_bytes;
  return AQP_OK;
}

extern "C" int aqp_cache_write(const aqp_cache_desc* desc, void* cache, const void* k, const void* v, int64_t num_tokens,
                               int64_t token_stride, const int64_t* slot_mapping, float k_scale, float v_scale,
                               void* stream) {
  if (!desc) return fail(AQP_ERR_INVALID, "aqp_cache_write: null descriptor");
  Geometry g;
  const char* why = "";
  int rc = make_geometry(*desc, &g, &why);
  if (rc) return fail(rc, "aqp_cache_write: %s", why);
  if (num_tokens < 0) return fail(AQP_ERR_INVALID, "aqp_cache_write: negative num_tokens");
  if (num_tokens == 0) return AQP_OK;
  if (!cache || !k || !v || !slot_mapping) return fail(AQP_ERR_INVALID, "aqp_cache_write: null pointer");
  if (token_stride < (int64_t)desc->num_kv_heads * desc->head_dim)
    return fail(AQP_ERR_INVALID, "aqp_cache_write: token_stride %lld < num_kv_heads * head_dim", (long long)token_stride);
  if (token_stride % 8 != 0 || ((uintptr_t)k % 16) || ((uintptr_t)v % 16))
    return fail(AQP_ERR_INVALID, "aqp_cache_write: k/v must be 16-byte aligned with a token_stride that is a multiple of 8");
  if (desc->mode == AQP_SCALE_PER_TENSOR && (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale < 0 || v_scale < 0))
    return fail(AQP_ERR_INVALID, "aqp_cache_write: per-tensor scales must be finite and non-negative");
  CacheWriteArgs a;
  a.cache = (uint8_t*)cache;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.token_stride = token_stride;
  a.page_bytes = g.page_bytes;
  a.block_bytes = g.block_bytes;
  a.total_slots = (int64_t)desc->num_blocks * desc->block_size;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.block_size = desc->block_size;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.narrow = 2 * num_tokens * desc->num_kv_heads < ((int64_t)1 << 31) && a.total_slots < ((int64_t)1 << 31) &&
             desc->num_kv_heads >= 2 && desc->block_size >= 2;
  a.heads_magic = a.bs_magic = 0;
  a.heads_shift = a.bs_shift = 0;
  if (a.narrow) {
    invariant_divisor((uint32_t)desc->num_kv_heads, &a.heads_magic, &a.heads_shift);
    invariant_divisor((uint32_t)desc->block_size, &a.bs_magic, &a.bs_shift);
  }
  return launch_cache_write(desc->dtype, desc->mode, a, stream);
}

// ---- schedule -------------------------------------------------------------

static int check_params(const aqp_attn_params& p, const aqp_cache_desc& d, const char** why) {
  if (p.num_kv_heads != d.num_kv_heads) { *why = "params.num_kv_heads differs from the cache's"; return AQP_ERR_INVALID; }
  if (p.head_dim != d.head_dim) { *why = "params.head_dim differs from the cache's"; return AQP_ERR_INVALID; }
  if (p.num_q_heads <= 0 || p.num_q_heads % p.num_kv_heads != 0) { *why = "num_q_heads must be a positive multiple of num_kv_heads"; return AQP_ERR_INVALID; }
  if (p.causal != 0 && p.causal != 1) { *why = "causal must be 0 or 1"; return AQP_ERR_INVALID; }
  if (p.window < 0) { *why = "negative window"; return AQP_ERR_INVALID; }
  if (p.window > 0 && !p.causal) { *why = "a sliding window needs causal attention"; return AQP_ERR_UNSUPPORTED; }
  if (p.max_blocks_per_seq <= 0) { *why = "max_blocks_per_seq must be positive"; return AQP_ERR_INVALID; }
  if (!(p.sm_scale >= 0.0f) || !std::isfinite(p.sm_scale)) { *why = "sm_scale must be finite and >= 0"; return AQP_ERR_INVALID; }
  if (!(p.softcap >= 0.0f) || !std::isfinite(p.softcap)) { *why = "softcap must be finite and >= 0"; return AQP_ERR_INVALID; }
  if (p.decode_parallelism < 0) { *why = "negative decode_parallelism"; return AQP_ERR_INVALID; }
  if (p.prefill_kv_split < 0) { *why = "negative prefill_kv_split"; return AQP_ERR_INVALID; }
  if (p.prefill_rows != 0 && p.prefill_rows != kPfRows && p.prefill_rows != kPfRowsSmall) { *why = "prefill_rows must be 0, 64 or 128"; return AQP_ERR_INVALID; }
  return AQP_OK;
}

static float effective_sm_scale(const aqp_attn_params& p) {
  return p.sm_scale > 0.0f ? p.sm_scale : (float)(1.0 / std::sqrt((double)p.head_dim));
}

extern "C" int aqp_get_schedule(const aqp_attn_params* params, const aqp_cache_desc* desc, const int32_t* seq_lens,
                                const int32_t* qsl, int32_t num_seqs, void* meta_host, size_t* meta_bytes,
                                size_t* scratch_bytes) {
  if (!params || !desc || !meta_bytes) return fail(AQP_ERR_INVALID, "aqp_get_schedule: null argument");
  if (num_seqs < 0) return fail(AQP_ERR_INVALID, "aqp_get_schedule: negative num_seqs");
  if (num_seqs > 0 && (!seq_lens || !qsl)) return fail(AQP_ERR_INVALID, "aqp_get_schedule: null seq_lens / query_start_loc");
  Geometry g;
  const char* why = "";
  int rc = make_geometry(*desc, &g, &why);
  if (rc) return fail(rc, "aqp_get_schedule: %s", why);
  rc = check_params(*params, *desc, &why);
  if (rc) return fail(rc, "aqp_get_schedule: %s", why);
  const aqp_attn_params& p = *params;
  const int32_t G = p.num_q_heads / p.num_kv_heads;
  const int32_t bs = desc->block_size;
  if (num_seqs > 0 && qsl[0] != 0) return fail(AQP_ERR_INVALID, "aqp_get_schedule: query_start_loc[0] must be 0");
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t L = seq_lens[b], ql = (int64_t)qsl[b + 1] - qsl[b];
    if (p.causal_per_seq) {
      const int32_t c = p.causal_per_seq[b];
      if (c != 0 && c != 1) return fail(AQP_ERR_INVALID, "aqp_get_schedule: causal_per_seq[%d] must be 0 or 1", b);
      if (c == 0 && p.window > 0) return fail(AQP_ERR_UNSUPPORTED, "aqp_get_schedule: a sliding window needs every sequence causal");
    }
    if (L < 0 || ql < 0 || ql > L)
      return fail(AQP_ERR_INVALID, "aqp_get_schedule: sequence %d has seq_len %lld and query_len %lld (need 0 <= query_len <= seq_len)", b, (long long)L, (long long)ql);
    if ((L + bs - 1) / bs > p.max_blocks_per_seq)
      return fail(AQP_ERR_INVALID, "aqp_get_schedule: sequence %d needs %lld blocks > max_blocks_per_seq %d", b, (long long)((L + bs - 1) / bs), p.max_blocks_per_seq);
  }
  const int64_t total_q = num_seqs > 0 ? qsl[num_seqs] : 0;
  if (total_q > INT32_MAX / 2) return fail(AQP_ERR_UNSUPPORTED, "aqp_get_schedule: too many query tokens");

  // ---- decode: units (sequence, KV head, head group) over their visible keys, laid end to end
  // and cut into equal runs of 16-key tiles, one run per work-group (one resident wave of them).
  struct Unit { int32_t seq, kvh, head0, nheads, lo, hi, q_tok; int64_t t0, ntiles; };
  // per-thread work buffers, reused across calls (the schedule is rebuilt every batch)
  static thread_local std::vector<Unit> units;
  static thread_local std::vector<DecSeg> segs;
  static thread_local std::vector<int32_t> wg_start;
  static thread_local std::vector<CombItem> comb;
  static thread_local std::vector<PfItem> pf;
  static thread_local std::vector<int32_t> unit_nseg, unit_first_part;
  units.clear();
  segs.clear();
  wg_start.clear();
  comb.clear();
  pf.clear();
  const int32_t max_hpu = heads_per_unit(desc->head_dim, g.kv_elem_bytes);
  const int32_t hpu = std::min<int32_t>(G, max_hpu);
  const int32_t dec_lds = dec_lds_bytes(desc->head_dim, desc->mode, hpu, g.kv_elem_bytes);
  if (dec_lds > kLdsPerCu) return fail(AQP_ERR_UNSUPPORTED, "aqp_get_schedule: decode needs %d bytes of LDS", dec_lds);
  int64_t total_tiles = 0, dec_keys = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t L = seq_lens[b], ql = qsl[b + 1] - qsl[b];
    if (ql != 1) continue;
    const int32_t pos = L - 1;
    const int32_t lo = (p.window > 0 && pos - p.window + 1 > 0) ? pos - p.window + 1 : 0;
    const int32_t hi = L;  // the single query sees every key up to its own position
    const int64_t t0 = lo / kTileKeys, t1 = (hi + kTileKeys - 1) / kTileKeys;
    for (int32_t h = 0; h < p.num_kv_heads; ++h) {
      dec_keys += hi - lo;
      for (int32_t h0 = 0; h0 < G; h0 += max_hpu) {
        units.push_back({b, h, h0, std::min<int32_t>(max_hpu, G - h0), lo, hi, qsl[b], t0, t1 - t0});
        total_tiles += t1 - t0;
      }
    }
  }
  int32_t num_parts = 0;
  int32_t num_wgs = 0;
  if (total_tiles > 0) {
    const int64_t target = p.decode_parallelism > 0 ? p.decode_parallelism
                                                    : (int64_t)device_cu_count() * decode_wgs_per_cu(desc->head_dim, dec_lds);
    const int64_t by_size = (total_tiles + kMinRunTiles - 1) / kMinRunTiles;
    int64_t P = std::max<int64_t>(1, std::min(target, by_size));
    const int64_t per = (total_tiles + P - 1) / P;
    P = (total_tiles + per - 1) / per;
    num_wgs = (int32_t)P;
    // first pass: count segments per unit to know which units are split
    unit_nseg.assign(units.size(), 0);
    {
      int64_t base = 0;
      for (size_t u = 0; u < units.size(); ++u) {
        const int64_t a = base, e = base + units[u].ntiles;
        unit_nseg[u] = (int32_t)((e - 1) / per - a / per + 1);
        base = e;
      }
    }
    unit_first_part.assign(units.size(), -1);
    for (size_t u = 0; u < units.size(); ++u) {
      if (unit_nseg[u] > 1) {
        unit_first_part[u] = num_parts;
        comb.push_back({units[u].kvh, units[u].head0, units[u].nheads, units[u].q_tok, num_parts * hpu, unit_nseg[u], hpu, 0});
        num_parts += unit_nseg[u];
      }
    }
    // second pass: emit segments grouped by work-group
    wg_start.assign(P + 1, 0);
    int64_t base = 0;
    int32_t w_cur = 0;
    for (size_t u = 0; u < units.size(); ++u) {
      const Unit& U = units[u];
      int64_t a = base;
      const int64_t e = base + U.ntiles;
      int32_t k = 0;
      while (a < e) {
        const int64_t w = a / per;
        const int64_t b_end = std::min(e, (w + 1) * per);
        while (w_cur < w) wg_start[++w_cur] = (int32_t)segs.size();
        const int64_t tile_lo = U.t0 + (a - base), tile_hi = U.t0 + (b_end - base);
        DecSeg s;
        s.seq = U.seq;
        s.kvh = U.kvh;
        s.head0 = U.head0;
        s.nheads = U.nheads;
        s.k_lo = (int32_t)std::max<int64_t>(U.lo, tile_lo * kTileKeys);
        s.k_hi = (int32_t)std::min<int64_t>(U.hi, tile_hi * kTileKeys);
        s.q_tok = U.q_tok;
        s.part = unit_nseg[u] > 1 ? unit_first_part[u] + k : -1;
        segs.push_back(s);
        ++k;
        a = b_end;
      }
      base = e;
    }
    while (w_cur < P) wg_start[++w_cur] = (int32_t)segs.size();
  }

  // ---- prefill items: (sequence, KV head, run of query tokens, run of its q heads): all G
  // heads of the KV head when G <= rows, else one token and `rows` heads at a time;
  // heaviest (most keys) first.
  auto build_items = [&](int32_t rows) {
    pf.clear();
    const int32_t hpi = std::min<int32_t>(G, rows);
    const int32_t tpi = std::max<int32_t>(1, rows / G);
    for (int32_t b = 0; b < num_seqs; ++b) {
      const int32_t L = seq_lens[b], ql = qsl[b + 1] - qsl[b];
      if (ql <= 1) continue;
      const int32_t causal = p.causal_per_seq ? p.causal_per_seq[b] : p.causal;
      for (int32_t q0 = 0; q0 < ql; q0 += tpi) {
        const int32_t q1 = std::min(ql, q0 + tpi);
        const int32_t khi = causal ? (L - ql + q1) : L;  // exclusive end of the last row's keys
        for (int32_t h = 0; h < p.num_kv_heads; ++h)
          for (int32_t h0 = 0; h0 < G; h0 += hpi)
            pf.push_back({b, h, q0, q1, L, ql, qsl[b], khi, h0, std::min(hpi, G - h0), causal, 0, khi, -1, 0, 0});
      }
    }
  };
  // first key of an item's key loop: the 16-key tile holding its first query's window start (the
  // prefill kernel starts its 32-key steps there)
  auto key_begin = [&](const PfItem& it) {
    const int32_t first = it.L - it.ql + it.q_lo;
    const int32_t lo = (p.window > 0 && first - p.window + 1 > 0) ? first - p.window + 1 : 0;
    return (lo / kTileKeys) * kTileKeys;
  };
  auto steps_of = [&](const PfItem& it) {
    const int32_t kb = std::max(key_begin(it), it.split_lo), ke = std::min(it.k_hi_max, it.split_hi);
    return ke > kb ? (ke - kb + kPfKvTile - 1) / kPfKvTile : 0;
  };
  // Key-split plan of the items in pf at `rows` rows per item: runs per item = its steps over the
  // target run length (the batch's steps spread over the work-groups the device holds), rounded to
  // nearest, at most max_runs, each run at least min_steps long. Split only when the batch has
  // fewer items than the device holds at once (or when the caller asks for it).
  struct SplitPlan { int32_t max_runs; int64_t min_steps, target; };
  auto split_plan = [&](int32_t rows) {
    SplitPlan sp{1, kPfMinSplitSteps, 1};
    int64_t total_steps = 0;
    for (const PfItem& it : pf) total_steps += steps_of(it);
    const int64_t cap = (int64_t)device_cu_count() *
                        (pf32_applies(desc->dtype, desc->mode, desc->head_dim, desc->block_size) ? pf32_wgs_per_cu(desc->head_dim, desc->mode, rows, g.pf_lds_bytes)
                                                               : pf_wgs_per_cu(desc->head_dim, rows, g.pf_lds_bytes));
    if (p.prefill_kv_split > 1) {
      sp.max_runs = p.prefill_kv_split;
      sp.min_steps = 1;
    } else if (p.prefill_kv_split == 0 && !pf.empty() && (int64_t)pf.size() < cap) {
      sp.max_runs = kPfMaxSplit;
      sp.target = std::max<int64_t>(1, (total_steps + cap - 1) / cap);
    }
    return sp;
  };
  auto runs_of = [&](const SplitPlan& sp, int32_t st) {
    if (sp.max_runs < 2) return 1;
    const int64_t want = (st + sp.target / 2) / sp.target;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>({(int64_t)sp.max_runs, want, st / sp.min_steps}));
  };
  // rows per item: kPfRows; at head_dim <= 128, for a batch with no decode work (decode runs beside
  // the prefill and needs the room a second work-group takes), kPfRowsSmall when kPfRows-row items,
  // even after key splits, would give the CUs fewer than two work-groups each. Per-group scales at
  // head_dim 128 take kPfRowsSmall always: the 128-row instance spills registers (4 x 512 and
  // 2 x 2048 token prefills measured 1.6-7 % faster with 64-row items)
  const bool pg128 = desc->mode == AQP_SCALE_PER_GROUP && desc->head_dim == 128;
  int32_t pf_rows = p.prefill_rows > 0 ? p.prefill_rows : (pg128 ? kPfRowsSmall : kPfRows);
  if (!pf32_applies(desc->dtype, desc->mode, desc->head_dim, desc->block_size) && pf_rows < pf_waves(desc->head_dim) * 16)
    return fail(AQP_ERR_UNSUPPORTED, "aqp_get_schedule: %d rows per prefill item at head_dim %d is not built", pf_rows, desc->head_dim);
  build_items(pf_rows);
  if (p.prefill_rows == 0 && !pg128 && desc->head_dim <= 128 && total_tiles == 0 && !pf.empty()) {
    const SplitPlan sp = split_plan(pf_rows);
    int64_t runs = 0;
    for (const PfItem& it : pf) runs += runs_of(sp, steps_of(it));
    if (runs < 2 * (int64_t)device_cu_count()) {
      pf_rows = kPfRowsSmall;
      build_items(pf_rows);
    }
  }
  // ---- prefill key splits: runs of whole 32-key steps; the rows of each run of a split item get
  // partial-result slots after the decode parts' (num_parts x hpu) slots, and each query token of
  // the item one merge item over its row in every run
  const int64_t num_dec_comb = (int64_t)comb.size();
  int64_t num_slots = (int64_t)num_parts * hpu;
  int64_t num_pf_split = 0;
  int32_t comb_heads = comb.empty() ? 0 : hpu;
  {
    const SplitPlan sp = split_plan(pf_rows);
    if (sp.max_runs > 1) {
      const size_t n0 = pf.size();
      for (size_t i = 0; i < n0; ++i) {
        const int32_t st = steps_of(pf[i]);
        const int32_t runs = runs_of(sp, st);
        if (runs < 2) continue;
        const PfItem base = pf[i];
        const int32_t kb = key_begin(base);
        const int32_t rows = (base.q_hi - base.q_lo) * base.nheads;
        const int64_t slot0 = num_slots;
        for (int32_t r = 0; r < runs; ++r) {
          PfItem it = base;
          it.split_lo = kb + (int32_t)((int64_t)st * r / runs) * kPfKvTile;
          it.split_hi = std::min(base.k_hi_max, kb + (int32_t)((int64_t)st * (r + 1) / runs) * kPfKvTile);
          it.slot = (int32_t)(slot0 + (int64_t)r * rows);
          if (r == 0) pf[i] = it; else pf.push_back(it);
        }
        for (int32_t t = base.q_lo; t < base.q_hi; ++t)
          comb.push_back({base.kvh, base.head0, base.nheads, base.q_start + t,
                          (int32_t)(slot0 + (int64_t)(t - base.q_lo) * base.nheads), runs, rows, 0});
        comb_heads = std::max(comb_heads, base.nheads);
        num_slots += (int64_t)runs * rows;
        num_pf_split += runs;
        if (num_slots > INT32_MAX / 2) return fail(AQP_ERR_UNSUPPORTED, "aqp_get_schedule: too many partial results");
      }
    }
  }
  // ---- order of the prefill items. The items of one (sequence, KV head) read the same K and V, and
  // work-group i runs on XCD i % kXcds, each XCD with an L2 of its own: so the items are packed into
  // kXcds bins of about equal work, a group at a time (largest first, a group larger than a bin's
  // share spilling into the next emptiest bin), so that a group's K and V are read into few L2s;
  // each bin's items run longest first, and the bins are interleaved into the launch order. Bins
  // short of items are padded with empty items (no rows and no keys: the kernels return at once).
  if (pf.size() >= (size_t)kXcds) {
    std::map<std::pair<int32_t, int32_t>, std::vector<size_t>> groups;
    for (size_t i = 0; i < pf.size(); ++i) groups[{pf[i].seq, pf[i].kvh}].push_back(i);
    auto work = [&](size_t i) { return std::max<int64_t>(1, steps_of(pf[i])); };
    std::vector<std::pair<int64_t, const std::vector<size_t>*>> order;
    int64_t total = 0;
    for (auto& g : groups) {
      int64_t w = 0;
      for (size_t i : g.second) w += work(i);
      total += w;
      order.push_back({w, &g.second});
    }
    std::stable_sort(order.begin(), order.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
    const int64_t share = (total + kXcds - 1) / kXcds;
    std::vector<int64_t> load(kXcds, 0);
    std::vector<std::vector<size_t>> bins(kXcds);
    auto emptiest = [&]() { return (int)(std::min_element(load.begin(), load.end()) - load.begin()); };
    for (auto& g : order) {
      std::vector<size_t> its = *g.second;
      std::stable_sort(its.begin(), its.end(), [&](size_t x, size_t y) { return work(x) > work(y); });
      int b = emptiest();
      for (size_t i : its) {
        if (load[b] > 0 && load[b] + work(i) > share) b = emptiest();
        bins[b].push_back(i);
        load[b] += work(i);
      }
    }
    size_t per = 0;
    for (auto& bn : bins) {
      std::stable_sort(bn.begin(), bn.end(), [&](size_t x, size_t y) { return work(x) > work(y); });
      per = std::max(per, bn.size());
    }
    PfItem empty{};
    empty.L = 1;
    empty.ql = 1;
    empty.nheads = 1;
    empty.slot = -1;
    std::vector<PfItem> out(per * kXcds, empty);
    for (int b = 0; b < kXcds; ++b)
      for (size_t j = 0; j < bins[b].size(); ++j) out[j * kXcds + b] = pf[bins[b][j]];
    pf.swap(out);
  } else if (pf.size() > 1) {
    std::stable_sort(pf.begin(), pf.end(), [&](const PfItem& x, const PfItem& y) { return steps_of(x) > steps_of(y); });
  }

  // ---- sizes and layout
  int64_t off = round_up(sizeof(SchedHeader), 256);
  const int64_t off_segs = off;
  off = round_up(off + (int64_t)segs.size() * sizeof(DecSeg), 256);
  const int64_t off_wgs = off;
  off = round_up(off + (int64_t)wg_start.size() * sizeof(int32_t), 256);
  // each decode work-group's first segment once more, indexed by work-group, so a work-group's
  // first copies wait on one record load instead of its range and then its segment
  const int64_t off_first = off;
  off = round_up(off + (int64_t)num_wgs * (int64_t)sizeof(DecSeg), 256);
  const int64_t off_comb = off;
  off = round_up(off + (int64_t)comb.size() * sizeof(CombItem), 256);
  const int64_t off_pf = off;
  off = round_up(off + (int64_t)pf.size() * sizeof(PfItem), 256);
  const int64_t off_sl = off;
  off = round_up(off + (int64_t)num_seqs * 4, 256);
  const int64_t need = off;
  const int64_t scratch = num_slots * slot_floats(desc->head_dim) * 4;
  if (scratch_bytes) *scratch_bytes = (size_t)scratch;
  if (!meta_host) { *meta_bytes = (size_t)need; return AQP_OK; }
  if (*meta_bytes < (size_t)need) {
    size_t have = *meta_bytes;
    *meta_bytes = (size_t)need;
    return fail(AQP_ERR_INVALID, "aqp_get_schedule: meta buffer of %zu bytes, need %lld", have, (long long)need);
  }
  *meta_bytes = (size_t)need;
  uint8_t* m = (uint8_t*)meta_host;
  // zero only the alignment gaps; every array byte is written below
  auto zero_gap = [&](int64_t from, int64_t to) { if (to > from) std::memset(m + from, 0, (size_t)(to - from)); };
  zero_gap(sizeof(SchedHeader), off_segs);
  zero_gap(off_segs + (int64_t)segs.size() * (int64_t)sizeof(DecSeg), off_wgs);
  zero_gap(off_wgs + (int64_t)wg_start.size() * 4, off_first);
  zero_gap(off_first + (int64_t)num_wgs * (int64_t)sizeof(DecSeg), off_comb);
  zero_gap(off_comb + (int64_t)comb.size() * (int64_t)sizeof(CombItem), off_pf);
  zero_gap(off_pf + (int64_t)pf.size() * (int64_t)sizeof(PfItem), off_sl);
  zero_gap(off_sl + (int64_t)num_seqs * 4, need);
  SchedHeader h;
  std::memset(&h, 0, sizeof h);
  h.magic = kMagic;
  h.version = kVersion;
  h.dtype = desc->dtype;
  h.mode = desc->mode;
  h.kv_elem_bytes = g.kv_elem_bytes;
  h.staged_elem_bytes = g.staged_elem_bytes;
  h.scale_bytes = g.scale_bytes;
  h.head_dim = desc->head_dim;
  h.block_size = desc->block_size;
  h.num_blocks = desc->num_blocks;
  h.num_q_heads = p.num_q_heads;
  h.num_kv_heads = p.num_kv_heads;
  h.causal = p.causal;
  h.window = p.window;
  h.max_blocks_per_seq = p.max_blocks_per_seq;
  h.num_seqs = num_seqs;
  h.sm_scale = effective_sm_scale(p);
  h.softcap = p.softcap;
  h.total_q_tokens = (int32_t)total_q;
  h.tile_keys = kTileKeys;
  h.dec_iter_keys = kDecIterKeys;
  h.dec_waves = kDecWaves;
  h.pf_rows = pf_rows;
  h.pf_kv_tile = kPfKvTile;
  h.heads_per_unit = max_hpu;
  h.dec_lds_bytes = dec_lds;
  h.pf_lds_bytes = g.pf_lds_bytes;
  h.num_dec_wgs = num_wgs;
  h.num_dec_segs = (int32_t)segs.size();
  h.num_parts = num_parts;
  h.num_comb = (int32_t)comb.size();
  h.num_pf_items = (int32_t)pf.size();
  h.group_heads = hpu;
  h.off_dec_segs = off_segs;
  h.off_dec_wg_start = off_wgs;
  h.off_dec_first = off_first;
  h.off_comb = off_comb;
  h.off_pf_items = off_pf;
  h.meta_bytes = need;
  h.scratch_bytes = scratch;
  h.page_bytes = g.page_bytes;
  h.block_bytes = g.block_bytes;
  h.dec_kv_keys = dec_keys;
  h.off_seq_lens = off_sl;
  h.num_slots = num_slots;
  h.comb_heads = comb_heads;
  h.num_pf_split = num_pf_split;
  h.num_dec_comb = num_dec_comb;
  std::memcpy(m, &h, sizeof h);
  if (!segs.empty()) std::memcpy(m + off_segs, segs.data(), segs.size() * sizeof(DecSeg));
  if (!wg_start.empty()) std::memcpy(m + off_wgs, wg_start.data(), wg_start.size() * sizeof(int32_t));
  for (int32_t w = 0; w < num_wgs; ++w) {
    DecSeg f;
    std::memset(&f, 0, sizeof f);
    if (wg_start[w] < wg_start[w + 1]) f = segs[wg_start[w]];
    std::memcpy(m + off_first + (int64_t)w * (int64_t)sizeof(DecSeg), &f, sizeof f);
  }
  if (!comb.empty()) std::memcpy(m + off_comb, comb.data(), comb.size() * sizeof(CombItem));
  if (!pf.empty()) std::memcpy(m + off_pf, pf.data(), pf.size() * sizeof(PfItem));
  if (num_seqs > 0) std::memcpy(m + off_sl, seq_lens, (size_t)num_seqs * 4);
  return AQP_OK;
}

// ---- attention -----------------------------------------------------------

#define MISMATCH_IF(cond, what)                                                      \
  do {                                                                               \
    if (cond) return fail(AQP_ERR_SCHEDULE_MISMATCH, "aqp_paged_attention: schedule was built for a different %s", what); \
  } while (0)

namespace aqp {

// The attention call on a given work buffer (`work`, `work_bytes` bytes).
static int attention(const aqp_attn_params* params, const aqp_cache_desc* desc, const void* cache, const void* q,
                     const int32_t* block_tables, const void* meta_host, const void* meta_dev, float k_scale,
                     float v_scale, void* work, size_t work_bytes, void* out, void* stream,
                     void* const* events = nullptr, int32_t num_events = 0) {
  if (!params || !desc || !meta_host) return fail(AQP_ERR_INVALID, "aqp_paged_attention: null argument");
  Geometry g;
  const char* why = "";
  int rc = make_geometry(*desc, &g, &why);
  if (rc) return fail(rc, "aqp_paged_attention: %s", why);
  rc = check_params(*params, *desc, &why);
  if (rc) return fail(rc, "aqp_paged_attention: %s", why);
  SchedHeader h;
  std::memcpy(&h, meta_host, sizeof h);
  if (h.magic != kMagic || h.version != kVersion) return fail(AQP_ERR_SCHEDULE_MISMATCH, "aqp_paged_attention: meta is not an aqp schedule of this version");
  // The schedule must describe exactly this cache and these parameters; its
  // element sizes and tile geometry must be the ones the kernels are built with.
  MISMATCH_IF(h.dtype != desc->dtype || h.mode != desc->mode, "kv dtype / scale mode");
  MISMATCH_IF(h.kv_elem_bytes != g.kv_elem_bytes || h.staged_elem_bytes != g.staged_elem_bytes || h.scale_bytes != g.scale_bytes, "KV element size");
  MISMATCH_IF(h.head_dim != desc->head_dim || h.block_size != desc->block_size || h.num_blocks != desc->num_blocks, "cache geometry");
  MISMATCH_IF(h.page_bytes != g.page_bytes || h.block_bytes != g.block_bytes, "page layout");
  MISMATCH_IF(h.num_q_heads != params->num_q_heads || h.num_kv_heads != params->num_kv_heads, "head count");
  MISMATCH_IF(h.causal != params->causal || h.window != params->window || h.max_blocks_per_seq != params->max_blocks_per_seq, "mask / block-table shape");
  MISMATCH_IF(h.sm_scale != effective_sm_scale(*params) || h.softcap != params->softcap, "logit scale / soft-cap");
  MISMATCH_IF(h.tile_keys != kTileKeys || h.dec_iter_keys != kDecIterKeys || h.dec_waves != kDecWaves || (h.pf_rows != kPfRows && h.pf_rows != kPfRowsSmall) ||
              (params->prefill_rows != 0 && h.pf_rows != params->prefill_rows) ||
              h.pf_kv_tile != kPfKvTile || h.heads_per_unit != heads_per_unit(desc->head_dim, g.kv_elem_bytes) ||
              h.dec_lds_bytes != dec_lds_bytes(desc->head_dim, desc->mode, std::min<int32_t>(params->num_q_heads / params->num_kv_heads, heads_per_unit(desc->head_dim, g.kv_elem_bytes)), g.kv_elem_bytes) ||
              h.pf_lds_bytes != g.pf_lds_bytes, "tile geometry");
  if ((int64_t)work_bytes < h.scratch_bytes)
    return fail(AQP_ERR_SCRATCH_TOO_SMALL, "aqp_paged_attention: scratch of %zu bytes, schedule needs %lld", work_bytes, (long long)h.scratch_bytes);
  if (h.scratch_bytes > 0 && !work) return fail(AQP_ERR_INVALID, "aqp_paged_attention: null scratch");
  if (h.total_q_tokens == 0) return AQP_OK;
  if (!cache || !q || !block_tables || !meta_dev || !out) return fail(AQP_ERR_INVALID, "aqp_paged_attention: null pointer");
  if (desc->mode == AQP_SCALE_PER_TENSOR && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
    return fail(AQP_ERR_INVALID, "aqp_paged_attention: per-tensor scales must be finite");
  AttnArgs a;
  a.cache = (const uint8_t*)cache;
  a.q = (const uint16_t*)q;
  a.block_tables = block_tables;
  a.meta_dev = (const uint8_t*)meta_dev;
  a.scratch = (float*)work;
  a.out = (uint16_t*)out;
  a.page_bytes = g.page_bytes;
  a.block_bytes = g.block_bytes;
  a.head_dim = desc->head_dim;
  a.block_size = desc->block_size;
  a.num_kv_heads = desc->num_kv_heads;
  a.num_q_heads = params->num_q_heads;
  a.group = params->num_q_heads / params->num_kv_heads;
  a.max_blocks_per_seq = params->max_blocks_per_seq;
  a.window = params->window;
  a.causal = params->causal;
  a.sm_scale = h.sm_scale;
  a.softcap = params->softcap;
  a.k_scale = desc->mode == AQP_SCALE_PER_TENSOR && desc->dtype != AQP_KV_AUTO ? k_scale : 1.0f;
  a.v_scale = desc->mode == AQP_SCALE_PER_TENSOR && desc->dtype != AQP_KV_AUTO ? v_scale : 1.0f;
  a.alibi_slopes = params->alibi_slopes;
  a.sinks = params->sinks;
  a.hdr = &h;
  // decode, then the merge of its split ranges; the prefill runs' merge follows the prefill
  const int32_t n_dec_comb = (int32_t)h.num_dec_comb, n_pf_comb = h.num_comb - n_dec_comb;
  auto launch_prefill_kernel = [&](void* st) -> int {
    return pf32_applies(desc->dtype, desc->mode, desc->head_dim, desc->block_size) ? launch_prefill32(desc->dtype, desc->mode, a, st)
                                                                                    : launch_prefill(desc->dtype, desc->mode, a, st);
  };
  // timing marks (aqp_paged_attention_timed): event i recorded on `stream` at point i
  auto mark = [&](int i) -> int {
    if (i >= num_events || !events || !events[i]) return AQP_OK;
    const hipError_t e = hipEventRecord((hipEvent_t)events[i], (hipStream_t)stream);
    return e == hipSuccess ? AQP_OK : fail(AQP_ERR_HIP, "aqp_paged_attention_timed: event %d: %s", i, hipGetErrorString(e));
  };
  // A mixed batch runs its decode and then its prefill on `stream`: the two kernels each fill the
  // device, and measured one after the other they finish sooner than side by side on two streams
  // (each takes the other's CUs and LDS).
  if ((rc = mark(0))) return rc;
  if (h.num_dec_segs > 0 && (rc = launch_decode(desc->dtype, desc->mode, a, stream))) return rc;
  if ((rc = mark(1))) return rc;
  if (h.num_dec_segs > 0 && n_dec_comb > 0 && (rc = launch_combine(a, 0, n_dec_comb, stream))) return rc;
  if ((rc = mark(2)) || (rc = mark(3))) return rc;
  if (h.num_pf_items > 0 && (rc = launch_prefill_kernel(stream))) return rc;
  if ((rc = mark(4))) return rc;
  if (h.num_pf_items > 0 && n_pf_comb > 0 && (rc = launch_combine(a, n_dec_comb, n_pf_comb, stream))) return rc;
  return mark(5);
}

// Scratch of the allocation-free call: a file-scope device array, one per GPU the library runs on,
// kept until the process ends. Host code never uses its name as an address (on the host the name is
// a stand-in, not device memory): the device address is taken once per device with
// hipGetSymbolAddress and used from then on.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Device address of this device's copy of `scratch` (taken on the first call on the device, with
// the device current), or null with the error set.
static void* noalloc_scratch() {
  static std::mutex mu;
  static void* per_dev[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    set_error("aqp_paged_attention_noalloc: no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!per_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      set_error("aqp_paged_attention_noalloc: hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
      return nullptr;
    }
    per_dev[dev] = p;
  }
  return per_dev[dev];
}

}  // namespace aqp

extern "C" int aqp_paged_attention(const aqp_attn_params* params, const aqp_cache_desc* desc, const void* cache,
                                   const void* q, const int32_t* block_tables, const void* meta_host,
                                   const void* meta_dev, float k_scale, float v_scale, void* scratch_buf,
                                   size_t scratch_bytes, void* out, void* stream) {
  return attention(params, desc, cache, q, block_tables, meta_host, meta_dev, k_scale, v_scale, scratch_buf,
                   scratch_bytes, out, stream);
}

extern "C" int aqp_paged_attention_timed(const aqp_attn_params* params, const aqp_cache_desc* desc, const void* cache,
                                         const void* q, const int32_t* block_tables, const void* meta_host,
                                         const void* meta_dev, float k_scale, float v_scale, void* scratch_buf,
                                         size_t scratch_bytes, void* out, void* stream, void* const* events,
                                         int32_t num_events) {
  if (num_events < 0 || (num_events > 0 && !events)) return fail(AQP_ERR_INVALID, "aqp_paged_attention_timed: bad event list");
  return attention(params, desc, cache, q, block_tables, meta_host, meta_dev, k_scale, v_scale, scratch_buf,
                   scratch_bytes, out, stream, events, std::min<int32_t>(num_events, 6));
}

extern "C" int aqp_paged_attention_noalloc(const aqp_attn_params* params, const aqp_cache_desc* desc,
                                           const void* cache, const void* q, const int32_t* block_tables,
                                           const void* meta_host, const void* meta_dev, float k_scale,
                                           float v_scale, void* out, void* stream) {
  if (!meta_host) return fail(AQP_ERR_INVALID, "aqp_paged_attention_noalloc: null argument");
  SchedHeader h;
  std::memcpy(&h, meta_host, sizeof h);
  // refused before any device call: a schedule whose partial results exceed the fixed buffer
  if (h.magic == kMagic && h.version == kVersion && h.scratch_bytes > (int64_t)kNoAllocScratchBytes)
    return fail(AQP_ERR_SCRATCH_TOO_SMALL,
                "aqp_paged_attention_noalloc: the schedule needs %lld bytes of scratch, the allocation-free call "
                "has a fixed %zu (use aqp_paged_attention with a caller buffer)",
                (long long)h.scratch_bytes, kNoAllocScratchBytes);
  void* work = h.scratch_bytes > 0 ? noalloc_scratch() : nullptr;
  if (h.scratch_bytes > 0 && !work) return AQP_ERR_HIP;
  return attention(params, desc, cache, q, block_tables, meta_host, meta_dev, k_scale, v_scale, work,
                   kNoAllocScratchBytes, out, stream);
}
