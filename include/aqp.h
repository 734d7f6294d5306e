/*
 * aqp -- quantized paged attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library (libaqp.so). Plain pointers and sizes only; every
 * device buffer is allocated and owned by the caller; the library allocates no
 * device memory at run time. State it keeps: a per-thread last-error message,
 * the compute-unit count of the first device it queried, and the device
 * address of its one static device array (the scratch of
 * aqp_paged_attention_noalloc: 64 MiB per GPU the library is loaded on, held
 * until the process ends).
 *
 * The operations follow three pages summarising vLLM pull requests:
 *  [P39445] "CPU backend adds FP8 KV-cache quantisation" (PR 39445)
 *  [P50194] "Fix CPU FP8 attention scheduler scratch sizing" (PR 50194)
 *  [P38378] "Per-token-head INT8/FP8 KV quantisation for Triton" (PR 38378)
 *
 * Conventions shared by every entry point:
 *  - Return value: an aqp_status; AQP_OK (0) or a negative code. On a
 *    negative code aqp_last_error() describes the failure and nothing was
 *    launched. There is no silent fallback to another precision or path: an
 *    unsupported combination is an error ([P39445] Motivation and
 *    Risk/Impact: the old silent downgrade to bf16 is what the pages remove).
 *  - Device work is enqueued asynchronously on `stream` (a hipStream_t; NULL
 *    is the default stream). Pointers named *_host are host memory; all other
 *    array pointers are device memory.
 *  - bf16 tensors are arrays of uint16 bit patterns.
 */
#ifndef AQP_H
#define AQP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* KV cache element type. Indices 0..2 are the kv_cache_dtype indices of
 * [P50194] Code excerpt (0 = auto, 1 = fp8_e4m3, 2 = fp8_e5m2); 3 adds int8
 * for the per-token-head mode of [P38378]. */
typedef enum {
  AQP_KV_AUTO = 0,     /* unquantised cache: the bf16 inputs stored as given, per-tensor mode, no scales */
  AQP_KV_FP8_E4M3 = 1, /* OCP E4M3, finite-only ("fn"), largest code 448 */
  AQP_KV_FP8_E5M2 = 2, /* OCP E5M2, largest finite code 57344 */
  AQP_KV_INT8 = 3      /* two's-complement int8, codes in [-128, 127] */
} aqp_kv_dtype;

/* Scale granularity ([P38378] Implementation item 1: the quantisation-mode
 * switch between per-tensor and per-token-head; its Risk/Impact names
 * per-group scales as a later addition without defining them: the reading
 * taken is AQP_SCALE_PER_GROUP). */
typedef enum {
  AQP_SCALE_PER_TENSOR = 0,     /* one k_scale and one v_scale, passed by the caller */
  AQP_SCALE_PER_TOKEN_HEAD = 1, /* one dynamic scale per (token, KV head), K and V apart, stored in the cache */
  AQP_SCALE_PER_GROUP = 2       /* one dynamic scale per (token, KV head, run of AQP_SCALE_GROUP consecutive
                                   head-dim channels), K and V apart, stored in the cache */
} aqp_scale_mode;
#define AQP_SCALE_GROUP 32

typedef enum {
  AQP_OK = 0,
  AQP_ERR_INVALID = -1,           /* null pointer, bad shape or value */
  AQP_ERR_UNSUPPORTED = -2,       /* valid request this build does not implement */
  AQP_ERR_SCHEDULE_MISMATCH = -3, /* schedule built for other parameters / element size */
  AQP_ERR_SCRATCH_TOO_SMALL = -4, /* scratch smaller than the schedule requires */
  AQP_ERR_HIP = -5                /* HIP runtime error (message has the HIP error string) */
} aqp_status;

/* Geometry of one paged KV cache allocation.
 *
 * Layout (the library's own; both the cache write and the attention kernels
 * use it, and the tests' reader follows the same definition):
 *  - num_blocks blocks, block b at byte b * block_bytes;
 *  - block_bytes = 2 * num_kv_heads * page_bytes: the K pages of heads
 *    0..Hkv-1, then the V pages;
 *  - a page holds block_size rows of head_dim codes (one byte each; two, the
 *    bf16 bits, for AUTO), token-major (row
 *    = one token of one head), followed in per-token-head mode by block_size
 *    fp32 scales (the scale of row r at page + block_size*head_dim + 4*r:
 *    the inline scale storage of [P38378] Implementation item 2, kept at the
 *    page tail so rows stay 16-byte aligned), in per-group mode by
 *    block_size * head_dim/32 fp32 scales (row r's group g at
 *    page + block_size*head_dim + 4*(r*head_dim/32 + g));
 *  - page_bytes is that content rounded up to a multiple of 128 bytes;
 *  - slot s is row (s % block_size) of block (s / block_size).
 * Supported: head_dim in {64, 128, 256} (every dtype and mode);
 * block_size from 1 to 65536 (a multiple of 16 keeps each 16-key tile in one
 * page; other sizes are gathered row by row). */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* aqp_kv_dtype */
  int32_t mode;  /* aqp_scale_mode */
} aqp_cache_desc;

/* Attention parameters ([P50194] Code excerpt: the scheduler's num_heads_q,
 * num_heads_kv, head_dim, causal, window_size, dynamic_causal; the harness's
 * soft_cap, use_alibi, use_sink). */
typedef struct {
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads; q head h reads KV head h / (Hq / Hkv) */
  int32_t num_kv_heads;       /* must equal the cache's */
  int32_t head_dim;           /* must equal the cache's */
  int32_t causal;             /* 1: query i of a sequence with L keys and ql queries sits at position
                                 L - ql + i and sees keys j <= that position; 0: sees all L keys */
  int32_t window;             /* 0: none; W > 0: only keys j with position - j < W (needs causal = 1) */
  int32_t max_blocks_per_seq; /* row stride of block_tables */
  float sm_scale;             /* logit scale; 0 means 1/sqrt(head_dim) */
  float softcap;              /* 0: none; c > 0: logit z -> c * tanh(z / c), applied after sm_scale */
  int32_t decode_parallelism; /* work-groups the decode work is split across; 0 = one resident wave of
                                 work-groups on the current device (CUs x 3 for head_dim <= 128, x 2 above) */
  int32_t prefill_rows;       /* query rows (token, q head) per prefill work-group: 64 or 128 (64 needs
                                 head_dim <= 128); 0 = 128, or 64 at head_dim <= 128 for a batch with no
                                 decode sequence whose 128-row items, after key splits, would number
                                 fewer than two per CU of the current device */
  /* The harness parameters the page names without defining them; the readings taken: */
  const int32_t* causal_per_seq; /* host int32 [num_seqs] of 0/1, or NULL (= `causal` for every
                                    sequence). Read by aqp_get_schedule only: the schedule carries
                                    each sequence's flag. A window needs every sequence causal. */
  const float* alibi_slopes;  /* device fp32 [num_q_heads], or NULL: the logit of key j for a query
                                 at position p gains slope[h] * (j - p), after the soft-cap. Read by
                                 aqp_paged_attention. */
  const float* sinks;         /* device fp32 [num_q_heads], or NULL: one more logit per q head in the
                                 softmax with no value row (it only enlarges the normaliser). Read
                                 by aqp_paged_attention. */
  int32_t prefill_kv_split;   /* key-range split of prefill work items ([P50194] Code excerpt:
                                 enable_kv_split): 0 = automatic (when the batch has fewer prefill
                                 items than the device runs at once, long items are cut into runs of
                                 at least 16 key steps of 32 keys, at most 8 runs, sized so the runs
                                 fill the device); 1 = never; n > 1 = every item with enough keys is
                                 cut into up to n runs. The runs' partial results are merged into
                                 the output like split decode ranges. */
} aqp_attn_params;

/* Parse a kv_cache_dtype string ([P50194] Code excerpt: parse_fp8_kv_dtype
 * maps the string to the dtype index; [P38378] Risk/Impact names the
 * per-token-head strings).
 *   "fp8", "fp8_e4m3"       -> FP8_E4M3, PER_TENSOR
 *   "fp8_e5m2"              -> FP8_E5M2, PER_TENSOR
 *   "int8_per_token_head"   -> INT8,     PER_TOKEN_HEAD
 *   "fp8_per_token_head"    -> FP8_E4M3, PER_TOKEN_HEAD
 * The two remaining codec x scale-mode pairs ([P38378] Risk/Impact: other
 * scale granularities are left as a later addition) have names of this
 * library's own:
 *   "int8"                  -> INT8,     PER_TENSOR
 *   "fp8_e5m2_per_token_head" -> FP8_E5M2, PER_TOKEN_HEAD
 *   "int8_per_group"        -> INT8,     PER_GROUP
 *   "fp8_per_group"         -> FP8_E4M3, PER_GROUP
 *   "fp8_e5m2_per_group"    -> FP8_E5M2, PER_GROUP
 *   "auto"                  -> AUTO,     PER_TENSOR (the unquantised cache)
 * Anything else: AQP_ERR_INVALID. Outputs are written only on AQP_OK. */
int aqp_parse_kv_dtype(const char* s, int32_t* dtype, int32_t* mode);

/* Byte sizes of the cache layout described at aqp_cache_desc. Any output
 * pointer may be NULL. Errors: INVALID / UNSUPPORTED for an unsupported
 * geometry. */
int aqp_cache_bytes(const aqp_cache_desc* desc, size_t* page_bytes, size_t* block_bytes, size_t* total_bytes);

/* Quantise new keys and values into the paged cache (reshape-and-cache with
 * quantisation: [P39445] Implementation items 1 and 3; [P38378]
 * Implementation item 3).
 *   k, v:          bf16 [num_tokens, Hkv, head_dim]; token t's head h starts at element
 *                  t * token_stride + h * head_dim (token_stride >= Hkv * head_dim).
 *   slot_mapping:  int64 [num_tokens]; slot < 0 means "do not store" (padding); slots
 *                  must be distinct; a slot >= num_blocks * block_size is not stored either.
 *   k_scale, v_scale: per-tensor mode only (ignored per token-head): dequantised
 *                  value = code * scale.
 * Per row (token, head, K or V), in fp32:
 *   s    = per tensor: the given scale; per token-head: max_d |x_d| / qmax
 *          (qmax = 448 for E4M3, 57344 for E5M2, 127 for INT8), stored inline; per
 *          group: the same over each run of AQP_SCALE_GROUP channels, one scale per run;
 *   inv  = (s == 0) ? 0 : 1 / s  (correctly rounded);
 *   code = fp8: round-to-nearest-even of x_d * inv, saturated to the largest finite code;
 *          int8: round-to-nearest-even, clamped to [-128, 127].
 * AUTO copies the bf16 values unchanged (no scale).
 * Errors: INVALID (null pointers, negative sizes, stride too small), UNSUPPORTED
 * (AUTO with a per-token-head or per-group mode), HIP. */
int aqp_cache_write(const aqp_cache_desc* desc, void* cache, const void* k, const void* v, int64_t num_tokens,
                    int64_t token_stride, const int64_t* slot_mapping, float k_scale, float v_scale, void* stream);

/* Build the per-batch attention schedule on the host ([P50194]
 * Implementation item 1 and Code excerpt: get_scheduler_metadata takes the
 * sequence lengths, query start locations, heads, head_dim, causal and window
 * flags and -- the fix -- the KV cache dtype, so that the tile geometry and the
 * scratch size are derived from the real KV element size).
 *   seq_lens_host:        int32 [num_seqs]: keys of each sequence (including its new tokens)
 *   query_start_loc_host: int32 [num_seqs + 1]: query tokens of sequence b are
 *                         [qsl[b], qsl[b+1]) of q / out; qsl[0] = 0; 0 <= ql <= L.
 *   meta_host:            output buffer of *meta_bytes bytes; NULL = size query only.
 *   meta_bytes:           in: capacity of meta_host; out: bytes needed/written.
 *   scratch_bytes:        out: device scratch aqp_paged_attention needs with this schedule.
 * Sequences with q_len == 1 become decode work, the others prefill work.
 * Decode key ranges are cut into equal runs of 16-key tiles, one per resident
 * work-group; prefill items (a run of query tokens times a run of one KV head's
 * q heads) may be cut into key runs (params->prefill_kv_split); split ranges
 * write partial results to the scratch, merged into the output in the same
 * call. The metadata is self-contained: it records the parameters and element sizes it
 * was built for, the geometry, and every work item. The caller copies the
 * meta_bytes bytes to device memory unchanged and passes both copies to
 * aqp_paged_attention.
 * Errors: INVALID, UNSUPPORTED. */
int aqp_get_schedule(const aqp_attn_params* params, const aqp_cache_desc* desc, const int32_t* seq_lens_host,
                     const int32_t* query_start_loc_host, int32_t num_seqs, void* meta_host, size_t* meta_bytes,
                     size_t* scratch_bytes);

/* Paged attention over the quantised cache with dequantisation fused into
 * the QK^T and PV products and an online softmax ([P39445] Implementation
 * item 2: the dequantise step inside the tile GEMMs, scale folding;
 * [P38378] Implementation item 3: dequantisation of KV tiles inside the
 * unified varlen attention).
 *   q:            bf16 [T_q, Hq, head_dim] contiguous, T_q = qsl[num_seqs].
 *   block_tables: int32 [num_seqs, max_blocks_per_seq]: physical block of each logical block.
 *                 Only the entries of blocks that hold a sequence's keys are read. An entry
 *                 outside [0, num_blocks) names no block: the keys of that logical block are
 *                 absent and take no part in the softmax (as if masked); the kernels read block
 *                 0 in its place and discard it, so no address leaves the cache. A row left with
 *                 no key and no sink is written as zeros.
 *   meta_host / meta_dev: the same schedule bytes, in host and device memory. The schedule
 *                 carries the batch's sequence lengths and query start locations (it was built
 *                 from them by aqp_get_schedule), so they are not passed again here.
 *   k_scale, v_scale: per-tensor mode only.
 *   scratch:      device buffer of at least the schedule's scratch_bytes (may be NULL if 0): the
 *                 partial results of split decode ranges and split prefill items.
 *   out:          bf16 [T_q, Hq, head_dim]; every row of every query token is written.
 * Per query row: z_j = sm_scale * q . k_j (k_j dequantised), soft-capped if
 * set, masked by causality and window; softmax over the visible keys; output
 * = sum_j p_j v_j rounded to bf16.
 * A batch with both decode and prefill sequences runs its decode kernels and
 * then its prefill kernels on `stream`; the work is complete when `stream`'s
 * work up to this call is.
 * Errors: INVALID, SCHEDULE_MISMATCH (schedule built for another cache
 * descriptor, dtype, element size or parameter set), SCRATCH_TOO_SMALL, HIP. */
int aqp_paged_attention(const aqp_attn_params* params, const aqp_cache_desc* desc, const void* cache,
                        const void* q, const int32_t* block_tables, const void* meta_host, const void* meta_dev,
                        float k_scale, float v_scale, void* scratch, size_t scratch_bytes, void* out, void* stream);

/* aqp_paged_attention for callers that time its kernels one by one (benchmarks, profilers that
 * read HIP events): identical work and results, and events[i] (hipEvent_t, or NULL to skip) is
 * recorded on `stream` at point i of the call: 0 before the decode kernel, 1 after it, 2 after the
 * merge of its split ranges, 3 before the prefill kernel, 4 after it, 5 after the merge of its
 * split runs. A part the batch does not have leaves its two points back to back. num_events: how
 * many entries `events` holds (0 to 6; more are ignored). The events belong to the caller and must
 * have been created on the stream's device. No event is recorded for a batch without query tokens
 * or when the call fails before its first launch.
 * Errors: those of aqp_paged_attention; INVALID for num_events < 0 or a null list with
 * num_events > 0; HIP when an event cannot be recorded. */
int aqp_paged_attention_timed(const aqp_attn_params* params, const aqp_cache_desc* desc, const void* cache,
                              const void* q, const int32_t* block_tables, const void* meta_host, const void* meta_dev,
                              float k_scale, float v_scale, void* scratch, size_t scratch_bytes, void* out,
                              void* stream, void* const* events, int32_t num_events);

/* aqp_paged_attention without a scratch argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * partial results of split ranges go to a fixed 64 MiB device array of the library (one per GPU
 * it runs on, held until the process ends; its address is looked up once per device on the
 * first call there). The call itself allocates nothing and creates nothing (the per-group
 * prefill kernels at head_dim 64 with 128-row items and at head_dim 256 spill registers: their
 * launches use the scratch memory the HIP runtime keeps for its queues). Arguments, layouts,
 * stream use and results are those of aqp_paged_attention. No part of the array has to
 * start at zero (every partial result is written before it is merged). Every call on one GPU
 * shares its array: calls that overlap on a GPU (other streams, other threads) race; serialise
 * them. Errors: those of aqp_paged_attention; SCRATCH_TOO_SMALL, before any device call, when
 * the schedule's scratch_bytes exceeds 64 MiB; HIP when the array's address cannot be read. */
int aqp_paged_attention_noalloc(const aqp_attn_params* params, const aqp_cache_desc* desc, const void* cache,
                                const void* q, const int32_t* block_tables, const void* meta_host,
                                const void* meta_dev, float k_scale, float v_scale, void* out, void* stream);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* aqp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AQP_H */
