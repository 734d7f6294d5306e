/*
 * CPU oracle for quantized paged attention -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct host implementation of what the GPU path
 * computes, used to check it. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library. It shares no code
 * with the HIP library: its own codec, its own cache-layout reader/writer and
 * its own attention loop.
 *
 * Sources (the pages are summaries of three vLLM pull requests):
 *  - "CPU backend adds FP8 KV-cache quantisation" (vllm PR 39445 page),
 *    Implementation items 1-3 and Review: scalar fp8 e4m3 quantise/dequantise,
 *    the e4m3fn / e5m2 formats, scale folding.
 *  - "Fix CPU FP8 attention scheduler scratch sizing" (vllm PR 50194 page),
 *    Code excerpt: the kv_cache_dtype indices 0 = auto, 1 = fp8_e4m3,
 *    2 = fp8_e5m2; the varlen paged harness parameters.
 *  - "Per-token-head INT8/FP8 KV quantisation for Triton" (vllm PR 38378 page),
 *    Implementation items 1-3 and Risk/Impact: dynamic per-(token, head)
 *    absmax scales stored inline with the data.
 *  - The OCP 8-bit floating point specification (OFP8, v1.0) for the bit-level
 *    definitions of E4M3 (finite-only "fn" variant) and E5M2.
 *
 * Floating point: the codec runs in fp32, the precision the quantised code is
 * decided in on the GPU; attention runs in fp64 over exactly-dequantised
 * values and rounds the result to bf16 once.
 */
#ifndef AQP_ORACLE_H
#define AQP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ORC_FMT_BF16: the unquantised cache ("auto" dtype): the bf16 inputs stored as given, two bytes
 * per element, per-tensor mode only (no scales). */
enum { ORC_FMT_BF16 = 0, ORC_FMT_E4M3 = 1, ORC_FMT_E5M2 = 2, ORC_FMT_INT8 = 3 };
/* ORC_MODE_PER_GROUP: one dynamic scale per (token, head, run of ORC_GROUP consecutive head-dim
 * channels), absmax / qmax like per-token-head: the per-group granularity the "Per-token-head
 * INT8/FP8 KV quantisation for Triton" page (Risk/Impact) names as a later addition without
 * defining it; the group width is this reading's choice. */
enum { ORC_MODE_PER_TENSOR = 0, ORC_MODE_PER_TOKEN_HEAD = 1, ORC_MODE_PER_GROUP = 2 };
enum { ORC_GROUP = 32 };

typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t fmt;  /* ORC_FMT_* */
  int32_t mode; /* ORC_MODE_* */
} orc_cache_desc;

int orc_num_threads(void);                          /* OpenMP threads the oracle runs with */

/* ---- codec ---- */
double orc_decode(int fmt, uint32_t code);          /* value of one code (NaN / inf where the format has them) */
uint32_t orc_encode(int fmt, float y);              /* fp8: RNE + satfinite; int8: RNE + clamp (two's complement byte) */
void orc_encode_array(int fmt, const float* y, int64_t n, uint8_t* out);
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f64_to_bf16(double x);                 /* round-to-nearest-even, once */
float orc_qmax(int fmt);                            /* 448, 57344, 127 */

/* ---- cache layout ---- */
int64_t orc_page_bytes(const orc_cache_desc* d);
int64_t orc_block_bytes(const orc_cache_desc* d);
int64_t orc_total_bytes(const orc_cache_desc* d);
/* Byte offset of page (block, kv in {0: K, 1: V}, head). */
int64_t orc_page_offset(const orc_cache_desc* d, int64_t block, int kv, int head);

/* ---- cache write: returns 0, or -1 on a slot outside the pool ---- */
int orc_cache_write(const orc_cache_desc* d, uint8_t* cache, const uint16_t* k, const uint16_t* v,
                    int64_t num_tokens, int64_t token_stride, const int64_t* slot_mapping,
                    float k_scale, float v_scale);

/* Dequantised row (D values, fp64) of K (kv = 0) or V (kv = 1) at (block, head, offset in block). */
void orc_read_row(const orc_cache_desc* d, const uint8_t* cache, int kv, int64_t block, int head,
                  int off, float k_scale, float v_scale, double* row);

/* ---- attention ----
 * q: bf16 [T_q, Hq, D]; out: bf16 [T_q, Hq, D]; out_f64 (optional): fp64 before rounding.
 * Returns 0 or -1 on invalid arguments. */
int orc_attention(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                  int32_t num_q_heads, int32_t causal, int32_t window, double sm_scale, double softcap,
                  float k_scale, float v_scale, uint16_t* out, double* out_f64);

/* Softmax weights of one query row (seq b, query i of that sequence, q head hq) over keys
 * [0, L); masked keys get 0. Returns 0 or -1. */
int orc_attention_weights(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t num_q_heads, int32_t causal, int32_t window, double sm_scale,
                          double softcap, float k_scale, float v_scale, int32_t b, int32_t i,
                          int32_t hq, double* w);

/* The same with the remaining parameters of the varlen harness of the "Fix CPU FP8 attention
 * scheduler scratch sizing" page (Code excerpt: dynamic_causal, use_alibi, use_sink), which the
 * page names without defining; the readings taken:
 *   causal_per_seq: int32 [num_seqs] (NULL: `causal` for every sequence): causal flag of each
 *                   sequence; a window needs causal sequences.
 *   alibi_slopes:   fp64 [Hq] (NULL: none): logit of key j for a query at position p gains
 *                   slope * (j - p), after the soft-cap.
 *   sinks:          fp64 [Hq] (NULL: none): one more logit per q head in the softmax, with no
 *                   value row (it only enlarges the normaliser). */
int orc_attention_ext(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                      int32_t num_q_heads, int32_t causal, const int32_t* causal_per_seq, int32_t window,
                      double sm_scale, double softcap, const double* alibi_slopes, const double* sinks,
                      float k_scale, float v_scale, uint16_t* out, double* out_f64);
int orc_attention_weights_ext(const orc_cache_desc* d, const uint8_t* cache, const uint16_t* q,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                              int32_t num_q_heads, int32_t causal, int32_t window, double sm_scale,
                              double softcap, double alibi_slope, double sink, float k_scale, float v_scale,
                              int32_t b, int32_t i, int32_t hq, double* w);

#ifdef __cplusplus
}
#endif
#endif
