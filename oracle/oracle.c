/*
 * CPU oracle for quantized paged attention -- TEST INFRASTRUCTURE ONLY.
 * Loaded by the test suite, the smoke check and the benchmark's CPU-baseline
 * leg; never by the library. See oracle.h for the sources followed.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off oracle.c -o liboracle.so -lm
 * (no fast-math: every fp32 step below must round exactly once, as written).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Format parameters, from the OCP 8-bit floating point definitions.        */
/*   E4M3 ("fn", finite): bias 7, 3 mantissa bits, no infinities,           */
/*        S.1111.111 is NaN, largest finite 448.                           */
/*   E5M2: bias 15, 2 mantissa bits, exponent 31 holds inf (m = 0) and      */
/*        NaN (m != 0), largest finite 57344.                               */
/* The "fn" / e5m2 pair is the one the PR 39445 page's review settles on    */
/* (the c10 Float8_e4m3fn / Float8_e5m2 types).                             */
/* ------------------------------------------------------------------------ */
typedef struct {
  int exp_bits, man_bits, bias;
  double max_finite;
} fp8_fmt;

static fp8_fmt fmt_of(int fmt) {
  fp8_fmt f;
  if (fmt == ORC_FMT_E4M3) { f.exp_bits = 4; f.man_bits = 3; f.bias = 7; f.max_finite = 448.0; }
  else { f.exp_bits = 5; f.man_bits = 2; f.bias = 15; f.max_finite = 57344.0; }
  return f;
}

float orc_qmax(int fmt) {
  if (fmt == ORC_FMT_INT8) return 127.0f;
  return (float)fmt_of(fmt).max_finite;
}

/* Decode: the bit-field closed form of the OCP definition. */
double orc_decode(int fmt, uint32_t code) {
  code &= 0xFFu;
  if (fmt == ORC_FMT_INT8) return (double)(int8_t)(uint8_t)code;
  fp8_fmt f = fmt_of(fmt);
  int sign = (code >> 7) & 1;
  int e = (int)((code >> f.man_bits) & ((1u << f.exp_bits) - 1));
  int m = (int)(code & ((1u << f.man_bits) - 1));
  double mag;
  if (fmt == ORC_FMT_E4M3 && e == 15 && m == 7) return NAN;
  if (fmt == ORC_FMT_E5M2 && e == 31) {
    if (m != 0) return NAN;
    return sign ? -INFINITY : INFINITY;
  }
  if (e == 0) mag = ldexp((double)m, 1 - f.bias - f.man_bits);             /* subnormal: m * 2^(1-bias-mbits) */
  else mag = ldexp(1.0 + (double)m / (double)(1 << f.man_bits), e - f.bias); /* normal */
  return sign ? -mag : mag;
}

/* Encode an fp32 value to fp8: round to nearest, ties to even, then saturate
 * to the largest finite magnitude ("satfinite"); infinities saturate too.
 * NaN maps to the format's canonical NaN (0x7F with the sign). */
static uint32_t enc_fp8(int fmt, float yf) {
  fp8_fmt f = fmt_of(fmt);
  double y = (double)yf; /* exact */
  uint32_t sign = signbit(y) ? 0x80u : 0u;
  if (isnan(y)) return sign | 0x7Fu;
  double a = fabs(y);
  int emin = 1 - f.bias; /* exponent of the smallest normal */
  double r;
  if (isinf(a)) r = f.max_finite;
  else {
    int ex;
    double quantum;
    if (a < ldexp(1.0, emin)) quantum = ldexp(1.0, emin - f.man_bits);
    else {
      (void)frexp(a, &ex);          /* a = fr * 2^ex, fr in [0.5, 1) */
      quantum = ldexp(1.0, (ex - 1) - f.man_bits);
    }
    r = nearbyint(a / quantum) * quantum; /* default rounding mode: ties to even; a/quantum is exact */
    if (r > f.max_finite) r = f.max_finite;
  }
  if (r == 0.0) return sign;
  /* r is now a representable magnitude: rebuild the bit fields. */
  uint32_t e_field, m_field;
  if (r < ldexp(1.0, emin)) {
    e_field = 0;
    m_field = (uint32_t)(r / ldexp(1.0, emin - f.man_bits));
  } else {
    int ex;
    double fr = frexp(r, &ex);      /* r = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;
    e_field = (uint32_t)(e + f.bias);
    m_field = (uint32_t)((fr * 2.0 - 1.0) * (double)(1 << f.man_bits));
  }
  return sign | (e_field << f.man_bits) | m_field;
}

/* int8: round to nearest, ties to even, clamp to [-128, 127]. NaN -> 0. */
static uint32_t enc_int8(float yf) {
  if (isnan(yf)) return 0;
  double r = nearbyint((double)yf);
  if (r > 127.0) r = 127.0;
  if (r < -128.0) r = -128.0;
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}

uint32_t orc_encode(int fmt, float y) {
  if (fmt == ORC_FMT_INT8) return enc_int8(y);
  return enc_fp8(fmt, y);
}

void orc_encode_array(int fmt, const float* y, int64_t n, uint8_t* out) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = (uint8_t)orc_encode(fmt, y[i]);
}

float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp64 -> bf16, one rounding (nearest, ties to even). bf16 keeps 8
 * significant bits and fp32's exponent range. */
uint16_t orc_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  double r;
  if (isinf(a)) r = INFINITY;
  else {
    double quantum;
    if (a < ldexp(1.0, -126)) quantum = ldexp(1.0, -133);
    else { int ex; (void)frexp(a, &ex); quantum = ldexp(1.0, (ex - 1) - 7); }
    r = nearbyint(a / quantum) * quantum;
    if (r > 3.3895313892515355e38) r = INFINITY; /* beyond the largest finite bf16 */
  }
  float rf = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &rf, 4);
  return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------------------ */
/* Cache layout.                                                             */
/* One allocation of num_blocks blocks. Block b holds 2*Hkv pages: first the */
/* K pages of heads 0..Hkv-1, then the V pages. A page holds block_size rows */
/* of head_dim code bytes, token-major; in per-token-head mode it is         */
/* followed by block_size fp32 scales (one per row: the "inline" scale of    */
/* the PR 38378 page); in per-group mode by block_size x head_dim/32 fp32    */
/* scales (row r's group g at index r * head_dim/32 + g). Each page is       */
/* padded to a multiple of 128 bytes.                                        */
/* ------------------------------------------------------------------------ */
/* Bytes per stored element: 2 for the unquantised bf16 cache, 1 for every code format. */
static int elem_bytes(int fmt) { return fmt == ORC_FMT_BF16 ? 2 : 1; }

int64_t orc_page_bytes(const orc_cache_desc* d) {
  int64_t content = (int64_t)d->block_size * d->head_dim * elem_bytes(d->fmt);
  if (d->mode == ORC_MODE_PER_TOKEN_HEAD) content += 4 * (int64_t)d->block_size;
  if (d->mode == ORC_MODE_PER_GROUP) content += 4 * (int64_t)d->block_size * (d->head_dim / ORC_GROUP);
  return (content + 127) / 128 * 128;
}
int64_t orc_block_bytes(const orc_cache_desc* d) { return 2 * (int64_t)d->num_kv_heads * orc_page_bytes(d); }
int64_t orc_total_bytes(const orc_cache_desc* d) { return (int64_t)d->num_blocks * orc_block_bytes(d); }
int64_t orc_page_offset(const orc_cache_desc* d, int64_t block, int kv, int head) {
  return block * orc_block_bytes(d) + ((int64_t)kv * d->num_kv_heads + head) * orc_page_bytes(d);
}

/* ------------------------------------------------------------------------ */
/* Cache write (reshape-and-cache with quantisation).                       */
/* Per token with a non-negative slot, per KV head, for K then V:           */
/*   x_d  = fp32(bf16 input)                                                 */
/*   s    = per-tensor: the given scale; per-token-head: max_d |x_d| / qmax  */
/*          (fp32 division), stored inline; per-group: the same over each    */
/*          run of ORC_GROUP consecutive d, one scale per run, stored inline */
/*   inv  = (s == 0) ? 0 : 1 / s   (fp32)                                    */
/*   code = encode(x_d * inv)      (fp32 product, then the format's rounding)*/
/* ------------------------------------------------------------------------ */
int orc_cache_write(const orc_cache_desc* d, uint8_t* cache, const uint16_t* k, const uint16_t* v,
                    int64_t num_tokens, int64_t token_stride, const int64_t* slot_mapping,
                    float k_scale, float v_scale) {
  const int64_t total_slots = (int64_t)d->num_blocks * d->block_size;
  const int D = d->head_dim, H = d->num_kv_heads, bs = d->block_size;
  const float qmax = orc_qmax(d->fmt);
  int bad = 0;
  int64_t t;
  for (t = 0; t < num_tokens; ++t)
    if (slot_mapping[t] >= total_slots) bad = 1;
  if (d->fmt == ORC_FMT_BF16 && d->mode != ORC_MODE_PER_TENSOR) bad = 1;
  if (d->mode == ORC_MODE_PER_GROUP && D % ORC_GROUP != 0) bad = 1;
  if (bad) return -1;
#pragma omp parallel for schedule(static)
  for (t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue; /* padding token: nothing stored */
    const int64_t block = slot / bs;
    const int off = (int)(slot % bs);
    for (int h = 0; h < H; ++h) {
      for (int kv = 0; kv < 2; ++kv) {
        const uint16_t* src = (kv == 0 ? k : v) + t * token_stride + (int64_t)h * D;
        uint8_t* page = cache + orc_page_offset(d, block, kv, h);
        if (d->fmt == ORC_FMT_BF16) { /* unquantised: the input row as given */
          memcpy(page + (int64_t)off * D * 2, src, (size_t)D * 2);
          continue;
        }
        if (d->mode == ORC_MODE_PER_GROUP) {
          const int ng = D / ORC_GROUP;
          for (int g = 0; g < ng; ++g) {
            float a = 0.0f;
            for (int i = g * ORC_GROUP; i < (g + 1) * ORC_GROUP; ++i) {
              float x = fabsf(orc_bf16_to_f32(src[i]));
              if (x > a) a = x;
            }
            const float sg = a / qmax;
            memcpy(page + (int64_t)bs * D + 4 * ((int64_t)off * ng + g), &sg, 4);
            const float inv = (sg == 0.0f) ? 0.0f : 1.0f / sg;
            for (int i = g * ORC_GROUP; i < (g + 1) * ORC_GROUP; ++i) {
              const float y = orc_bf16_to_f32(src[i]) * inv;
              page[(int64_t)off * D + i] = (uint8_t)orc_encode(d->fmt, y);
            }
          }
          continue;
        }
        float s;
        if (d->mode == ORC_MODE_PER_TOKEN_HEAD) {
          float a = 0.0f;
          for (int i = 0; i < D; ++i) {
            float x = fabsf(orc_bf16_to_f32(src[i]));
            if (x > a) a = x;
          }
          s = a / qmax;
          memcpy(page + (int64_t)bs * D + 4 * (int64_t)off, &s, 4);
        } else {
          s = (kv == 0) ? k_scale : v_scale;
        }
        const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
        for (int i = 0; i < D; ++i) {
          const float y = orc_bf16_to_f32(src[i]) * inv;
          page[(int64_t)off * D + i] = (uint8_t)orc_encode(d->fmt, y);
        }
      }
    }
  }
  return 0;
}

/* Dequantised value = decode(code) * scale: the scale is a multiplier, the
 * same meaning as on the GPU backend (PR 39445 page, Risk/Impact). In fp64
 * the product is exact. */
void orc_read_row(const orc_cache_desc* d, const uint8_t* cache, int kv, int64_t block, int head,
                  int off, float k_scale, float v_scale, double* row) {
  const int D = d->head_dim;
  const uint8_t* page = cache + orc_page_offset(d, block, kv, head);
  if (d->fmt == ORC_FMT_BF16) {
    uint16_t w;
    for (int i = 0; i < D; ++i) {
      memcpy(&w, page + ((int64_t)off * D + i) * 2, 2);
      row[i] = (double)orc_bf16_to_f32(w);
    }
    return;
  }
  if (d->mode == ORC_MODE_PER_GROUP) {
    const int ng = D / ORC_GROUP;
    for (int i = 0; i < D; ++i) {
      float sf;
      memcpy(&sf, page + (int64_t)d->block_size * D + 4 * ((int64_t)off * ng + i / ORC_GROUP), 4);
      row[i] = orc_decode(d->fmt, page[(int64_t)off * D + i]) * (double)sf;
    }
    return;
  }
  double s;
  if (d->mode == ORC_MODE_PER_TOKEN_HEAD) {
    float sf;
    memcpy(&sf, page + (int64_t)d->block_size * D + 4 * (int64_t)off, 4);
    s = (double)sf;
  } else {
    s = (double)(kv == 0 ? k_scale : v_scale);
  }
  for (int i = 0; i < D; ++i) row[i] = orc_decode(d->fmt, page[(int64_t)off * D + i]) * s;
}

/* ------------------------------------------------------------------------ */
/* Attention: the plain definition, in fp64.                                 */
/* Sequence b has L = seq_lens[b] keys and ql = qsl[b+1] - qsl[b] queries;   */
/* query i sits at absolute position p = L - ql + i (the (query_len,         */
/* kv_len) tuples of the PR 50194 page's varlen harness: the queries are the */
/* newest ql positions). q head hq reads KV head hq / (Hq / Hkv).            */
/* Visible keys: j <= p when causal (all j < L otherwise), and p - j < W     */
/* when a window W > 0 is set.                                               */
/*   z_j = sm_scale * q . k_j ;  z_j = cap * tanh(z_j / cap) if cap > 0      */
/*   w_j = exp(z_j - max z) / sum ;  o = sum_j w_j v_j ;  out = bf16(o)       */
/* ------------------------------------------------------------------------ */
typedef struct {
  const orc_cache_desc* d;
  const uint8_t* cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  float k_scale, v_scale;
} orc_ctx;

static int check_args(const orc_cache_desc* d, const int32_t* seq_lens, const int32_t* qsl, int32_t num_seqs,
                      int32_t Hq, int32_t causal, const int32_t* causal_per_seq, int32_t window, int32_t max_blocks) {
  if (d->num_kv_heads <= 0 || Hq <= 0 || Hq % d->num_kv_heads != 0) return -1;
  if (window < 0 || (window > 0 && !causal)) return -1;
  for (int b = 0; b < num_seqs; ++b) {
    if (causal_per_seq && window > 0 && !causal_per_seq[b]) return -1;
    int32_t L = seq_lens[b], ql = qsl[b + 1] - qsl[b];
    if (ql < 0 || L < ql || (ql > 0 && L == 0)) return -1;
    if (((int64_t)L + d->block_size - 1) / d->block_size > max_blocks) return -1;
  }
  return 0;
}

/* Gather dequantised K and V rows [lo, L) of (b, kvh) into kk, vv ([n][D]). A key whose
 * block-table entry lies outside the pool [0, num_blocks) has no row to read: its flag in
 * `present` is 0 and its rows are zeros; such keys take no part in the softmax (reading: a
 * table entry that names no block of the pool marks that block's keys as absent, the same as
 * a masked key). */
static void gather(const orc_ctx* c, int b, int kvh, int32_t lo, int32_t L, double* kk, double* vv,
                   unsigned char* present) {
  const orc_cache_desc* d = c->d;
  for (int32_t j = lo; j < L; ++j) {
    int32_t blk = c->block_tables[(int64_t)b * c->max_blocks + j / d->block_size];
    double* kr = kk + (int64_t)(j - lo) * d->head_dim;
    double* vr = vv + (int64_t)(j - lo) * d->head_dim;
    present[j - lo] = blk >= 0 && blk < d->num_blocks;
    if (!present[j - lo]) {
      for (int dd = 0; dd < d->head_dim; ++dd) kr[dd] = vr[dd] = 0.0;
      continue;
    }
    int off = j % d->block_size;
    orc_read_row(d, c->cache, 0, blk, kvh, off, c->k_scale, c->v_scale, kr);
    orc_read_row(d, c->cache, 1, blk, kvh, off, c->k_scale, c->v_scale, vr);
  }
}

static void key_range(int32_t L, int32_t ql, int32_t i, int32_t causal, int32_t window, int32_t* lo, int32_t* hi) {
  int32_t p = L - ql + i;
  *hi = causal ? p : L - 1;
  *lo = (window > 0 && p - window + 1 > 0) ? p - window + 1 : 0;
}

/* Weights of one row (query at position p) over the gathered keys [lo0, ...): w has (L - lo0)
 * entries. Logit of key j: z = sm_scale * q.k_j, soft-capped (cap * tanh(z / cap)) if cap > 0,
 * plus the linear position bias slope * (j - p) (ALiBi; slope 0 = none). The softmax runs over
 * the visible keys that are present (see gather) and, if sink is finite, one more logit `sink`
 * that has no value row: it only adds exp(sink - m) to the normaliser, so the key weights sum to
 * less than one. A row left with no key and no sink has all weights 0 (its output is 0). */
static void row_weights(const double* qrow, const double* kk, const unsigned char* present, int32_t lo0,
                        int32_t lo, int32_t hi, int D, double sm_scale, double softcap, double slope, int32_t p,
                        double sink, double* w, int32_t n) {
  double m = sink;  /* -inf when there is no sink */
  for (int32_t j = 0; j < n; ++j) w[j] = 0.0;
  for (int32_t j = lo; j <= hi; ++j) {
    if (!present[j - lo0]) continue;
    const double* kr = kk + (int64_t)(j - lo0) * D;
    double dot = 0.0;
    for (int dd = 0; dd < D; ++dd) dot += qrow[dd] * kr[dd];
    double z = sm_scale * dot;
    if (softcap > 0.0) z = softcap * tanh(z / softcap);
    z += slope * (double)(j - p);
    w[j - lo0] = z;
    if (z > m) m = z;
  }
  if (isinf(m) && m < 0) {  /* nothing to attend to */
    for (int32_t j = 0; j < n; ++j) w[j] = 0.0;
    return;
  }
  double l = isinf(sink) ? 0.0 : exp(sink - m);
  for (int32_t j = lo; j <= hi; ++j) {
    if (!present[j - lo0]) continue;
    w[j - lo0] = exp(w[j - lo0] - m);
    l += w[j - lo0];
  }
  for (int32_t j = lo; j <= hi; ++j) w[j - lo0] /= l;
}

int orc_attention(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                  int32_t num_q_heads, int32_t causal, int32_t window, double sm_scale, double softcap,
                  float k_scale, float v_scale, uint16_t* out, double* out_f64) {
  return orc_attention_ext(d, cache, q, block_tables, max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                           num_q_heads, causal, NULL, window, sm_scale, softcap, NULL, NULL, k_scale, v_scale, out,
                           out_f64);
}

int orc_attention_ext(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                      int32_t num_q_heads, int32_t causal, const int32_t* causal_per_seq, int32_t window,
                      double sm_scale, double softcap, const double* alibi_slopes, const double* sinks,
                      float k_scale, float v_scale, uint16_t* out, double* out_f64) {
  if (check_args(d, seq_lens, query_start_loc, num_seqs, num_q_heads, causal, causal_per_seq, window,
                 max_blocks_per_seq)) return -1;
  const int D = d->head_dim, Hkv = d->num_kv_heads, Hq = num_q_heads, G = Hq / Hkv;
  if (sm_scale <= 0.0) sm_scale = 1.0 / sqrt((double)D);
  orc_ctx c = {d, cache, block_tables, max_blocks_per_seq, k_scale, v_scale};
  int failed = 0;
  int64_t task;
  const int64_t ntasks = (int64_t)num_seqs * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (task = 0; task < ntasks; ++task) {
    const int b = (int)(task / Hkv), kvh = (int)(task % Hkv);
    const int32_t L = seq_lens[b], ql = query_start_loc[b + 1] - query_start_loc[b];
    if (ql == 0) continue;
    const int32_t cz = causal_per_seq ? causal_per_seq[b] : causal;
    int32_t lo0, hi0;
    key_range(L, ql, 0, cz, window, &lo0, &hi0);
    const int32_t n = L - lo0;
    double* kk = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* vv = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* w = (double*)malloc(sizeof(double) * (size_t)n);
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
    unsigned char* present = (unsigned char*)malloc((size_t)(n > 0 ? n : 1));
    if (!kk || !vv || !w || !qrow || !o || !present) {
#pragma omp atomic write
      failed = 1;
    } else {
      gather(&c, b, kvh, lo0, L, kk, vv, present);
      for (int32_t i = 0; i < ql; ++i) {
        int32_t lo, hi;
        key_range(L, ql, i, cz, window, &lo, &hi);
        const int64_t tok = (int64_t)query_start_loc[b] + i;
        for (int g = 0; g < G; ++g) {
          const int hq = kvh * G + g;
          const uint16_t* qsrc = q + (tok * Hq + hq) * D;
          for (int dd = 0; dd < D; ++dd) qrow[dd] = (double)orc_bf16_to_f32(qsrc[dd]);
          row_weights(qrow, kk, present, lo0, lo, hi, D, sm_scale, softcap, alibi_slopes ? alibi_slopes[hq] : 0.0,
                      L - ql + i, sinks ? sinks[hq] : -INFINITY, w, n);
          for (int dd = 0; dd < D; ++dd) o[dd] = 0.0;
          for (int32_t j = lo; j <= hi; ++j) {
            const double wj = w[j - lo0];
            const double* vr = vv + (int64_t)(j - lo0) * D;
            for (int dd = 0; dd < D; ++dd) o[dd] += wj * vr[dd];
          }
          for (int dd = 0; dd < D; ++dd) {
            out[(tok * Hq + hq) * D + dd] = orc_f64_to_bf16(o[dd]);
            if (out_f64) out_f64[(tok * Hq + hq) * D + dd] = o[dd];
          }
        }
      }
    }
    free(kk); free(vv); free(w); free(qrow); free(o); free(present);
  }
  return failed ? -1 : 0;
}

int orc_attention_weights(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t num_q_heads, int32_t causal, int32_t window, double sm_scale,
                          double softcap, float k_scale, float v_scale, int32_t b, int32_t i,
                          int32_t hq, double* w) {
  return orc_attention_weights_ext(d, cache, q, block_tables, max_blocks_per_seq, seq_lens, query_start_loc,
                                   num_seqs, num_q_heads, causal, window, sm_scale, softcap, 0.0, -INFINITY,
                                   k_scale, v_scale, b, i, hq, w);
}

int orc_attention_weights_ext(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                              int32_t num_q_heads, int32_t causal, int32_t window, double sm_scale,
                              double softcap, double alibi_slope, double sink, float k_scale, float v_scale,
                              int32_t b, int32_t i, int32_t hq, double* w) {
  if (check_args(d, seq_lens, query_start_loc, num_seqs, num_q_heads, causal, NULL, window, max_blocks_per_seq))
    return -1;
  if (b < 0 || b >= num_seqs || hq < 0 || hq >= num_q_heads) return -1;
  const int D = d->head_dim, Hkv = d->num_kv_heads, G = num_q_heads / Hkv;
  const int32_t L = seq_lens[b], ql = query_start_loc[b + 1] - query_start_loc[b];
  if (i < 0 || i >= ql) return -1;
  if (sm_scale <= 0.0) sm_scale = 1.0 / sqrt((double)D);
  orc_ctx c = {d, cache, block_tables, max_blocks_per_seq, k_scale, v_scale};
  int32_t lo, hi;
  key_range(L, ql, i, causal, window, &lo, &hi);
  double* kk = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * D);
  double* vv = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * D);
  double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
  unsigned char* present = (unsigned char*)malloc((size_t)(L > 0 ? L : 1));
  int rc = -1;
  if (kk && vv && qrow && present) {
    gather(&c, b, hq / G, 0, L, kk, vv, present);
    const int64_t tok = (int64_t)query_start_loc[b] + i;
    for (int dd = 0; dd < D; ++dd) qrow[dd] = (double)orc_bf16_to_f32(q[(tok * num_q_heads + hq) * D + dd]);
    row_weights(qrow, kk, present, 0, lo, hi, D, sm_scale, softcap, alibi_slope, L - ql + i, sink, w, L);
    rc = 0;
  }
  free(kk); free(vv); free(qrow); free(present);
  return rc;
}
