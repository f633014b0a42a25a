/*
 * kvq.h -- C ABI of libkvq: quantized KV-cache append and decode attention on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes is defined by these pages:
 *   [I]  ORT issue "Feature request: quantized (int8/fp8) KV cache in
 *        GroupQueryAttention with past/present shared buffer + CUDA graph capture"
 *   [P]  ORT PR "[CUDA] PagedAttention: quantized KV cache, XQA decode, MLA,
 *        QK-Norm and head sink"
 *   [F]  ORT PR "[CUDA] Add INT4 paged KV cache with per-channel scales"
 *   [K]  kernel page "kv-quant-attn"
 *
 * Conventions that hold for every call below:
 *   - Every pointer argument is a DEVICE pointer unless it is marked "host".
 *     The caller owns every buffer (cache, scales, workspace, outputs); the
 *     library allocates nothing, keeps no state between calls and holds no
 *     handles, so calls from different host threads on different streams are
 *     safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A
 *     call only enqueues work on it: no host synchronization, no allocation and
 *     no host read of device data, so every call can be captured into a HIP
 *     graph ([P] Summary of Changes, the CUDA-graph-safety bullet: grid sizes
 *     and workspace extents come from static shapes and a host capacity bound,
 *     per-step quantities are read on the device).
 *   - Return value: KVQ_OK or a negative kvq_status.  Argument errors are
 *     detected on the host before anything is enqueued; nothing is launched
 *     then.  KVQ_EHIP reports a launch failure returned by the HIP runtime.
 *     No C++ exception crosses this interface.
 *   - Activations (k, v, q, out) are bf16, passed as raw 16-bit patterns.
 *
 * Data layout of a cache (one layer, one side each for K and V):
 *   codes   [num_blocks, num_kv_heads, block_size, row_bytes] bytes, where
 *           row_bytes = head_dim for int8 / fp8 and head_dim / 2 for int4
 *           (two signed 4-bit values per byte, element 2i in the low nibble);
 *           2 * head_dim for the unquantized bf16 cache (the values themselves)
 *   scales  KVQ_PER_ROW:     fp32 [num_blocks, num_kv_heads, block_size],
 *                            written by kvq_append next to each row
 *           KVQ_PER_TENSOR:  fp32 [1], static, filled by the caller
 *           KVQ_PER_CHANNEL: fp32 [num_kv_heads, head_dim], static
 *   Token p of sequence b lives in block block_table[b * max_blocks + p /
 *   block_size] at row p % block_size.  The contiguous cache [B, Hkv, T, D] of
 *   [I] ("Motivation": one fixed-capacity buffer bound as past and present) is
 *   the case num_blocks = B, block_size = T (the capacity), no block table:
 *   sequence b owns block b.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache element types: [P] T_CACHE (int8, float8e4m3fn); [F] packed int4.
 * KVQ_BF16 is the unquantized cache the quantized ones are measured against
 * ([K] "Performance": int8 decode against a bf16 cache): rows hold the bf16
 * values as appended, there are no scales (scale_mode and v_scale_mode must be
 * KVQ_NO_SCALE; k_scales / v_scales are never read and may be NULL), and the
 * decode is exact attention over those values. */
typedef enum kvq_dtype {
  KVQ_INT8 = 1,       /* signed, symmetric grid [-127, 127] */
  KVQ_INT4 = 2,       /* signed, symmetric grid [-7, 7], two per byte */
  KVQ_FP8_E4M3FN = 3, /* OCP E4M3, no infinities, saturating at +-448 */
  KVQ_BF16 = 4        /* unquantized bf16 rows */
} kvq_dtype;

/* Scale granularity: per row ([K] "Method": every K and V row carries its own
 * absmax scale, computed when written); per tensor / per channel ([P] the
 * k_scale / v_scale inputs with PER_TENSOR | PER_CHANNEL quant types). */
typedef enum kvq_scale_mode {
  KVQ_NO_SCALE = 0, /* KVQ_BF16 only */
  KVQ_PER_ROW = 1,
  KVQ_PER_TENSOR = 2,
  KVQ_PER_CHANNEL = 3
} kvq_scale_mode;

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,       /* null required pointer, inconsistent sizes, workspace too small */
  KVQ_EUNSUPPORTED = -2, /* head_dim not in {64,128,256}, Hq/Hkv > 8, q_tokens > 8, unknown enum */
  KVQ_EHIP = -3,         /* the HIP runtime reported a launch error */
  KVQ_ESCRATCH = -4      /* kvq_attend_ex_noalloc: the call needs more workspace than
                            KVQ_NOALLOC_SCRATCH_BYTES */
} kvq_status;

/* One layer's quantized cache.  K and V share the dtype; scale_mode is the K
 * side's scale mode and v_scale_mode the V side's (0: the same as scale_mode;
 * [P]: k_scale and v_scale are separate inputs).  k_scales / v_scales point at
 * the per-row arrays (KVQ_PER_ROW, written by kvq_append) or at the static
 * tables (KVQ_PER_TENSOR [1], KVQ_PER_CHANNEL [num_kv_heads, head_dim]), which
 * must be finite and >= 0; a zero static scale stores code 0. */
typedef struct kvq_cache {
  int32_t dtype;        /* kvq_dtype */
  int32_t scale_mode;   /* kvq_scale_mode */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* D in {64, 128, 256} */
  int32_t block_size;   /* tokens per block, a positive multiple of 16 */
  int32_t num_blocks;   /* blocks in the pool (B for a contiguous cache) */
  void* k_codes;
  void* v_codes;
  float* k_scales;
  float* v_scales;
  int32_t v_scale_mode; /* kvq_scale_mode of V, or 0: as scale_mode */
} kvq_cache;

/*
 * Options of kvq_attend_ex ([P] "CUDA kernels": the paged decode kernel takes a
 * logit soft cap and a sliding window).
 *   softcap  > 0: every scaled logit z = softmax_scale * q . k becomes
 *            softcap * tanh(z / softcap) before the softmax (the head-sink logit is
 *            not capped); 0: off.  Finite, >= 0.
 *   window   > 0: the query at position p attends only the tokens
 *            p - window + 1 .. p (with the causal bound of speculative drafts);
 *            whole 16-token tiles before the first query's window are not read.
 *            0: every cached token.
 */
typedef struct kvq_attn_options {
  float softcap;
  int32_t window;
} kvq_attn_options;

/*
 * kvq_append -- quantize `tokens` new K and V rows per sequence on write and
 * store them at positions positions[b] + j (j < tokens).
 *
 *   k, v        bf16 [batch, tokens, num_kv_heads, head_dim]
 *   positions   int32 [batch]: first position written for each sequence
 *   block_table int32 [batch, max_blocks], or NULL for the contiguous cache
 *
 * Per row ([K] "Method"; [I] "Motivation": appending never re-quantizes
 * earlier entries): PER_ROW takes s = max|x| / Qmax (IEEE fp32 division; Qmax
 * 127 int8, 7 int4, 448 fp8) and stores it; static modes use the given scale.
 * Each code is the nearest grid value to x / s (fp32 division), ties to even,
 * clamped to [-Qmax, Qmax] (fp8 saturates at +-448 and keeps the sign of
 * zero); s == 0 gives code 0.  Only the addressed rows and their scales are
 * written ([P] "CUDA kernels": ReshapeAndCache quantizes on write).  A
 * KVQ_BF16 cache stores the rows as given.
 * Device-side preconditions (not checked on the host, which never reads
 * device data): rows whose position falls outside the sequence's capacity or
 * whose block_table entry is outside [0, num_blocks) are skipped.
 */
int kvq_append(const kvq_cache* cache, const void* k, const void* v, int32_t batch,
               int32_t tokens, const int32_t* positions, const int32_t* block_table,
               int32_t max_blocks, void* stream);

/*
 * kvq_num_splits -- the decode's split divisor W for a shape: the tiles of
 * all sequences are cut into chunks of C = max(ceil(T / W), 8) tiles (T = the
 * 16-token tiles of the batch), so a single sequence of max_seq_len tokens is
 * read by W workgroups per KV head.  A pure function of its (host) arguments,
 * so a captured graph and the workspace size stay valid for every step that
 * keeps the same bound.
 */
int32_t kvq_num_splits(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                       int32_t q_tokens, int32_t max_seq_len);

/*
 * kvq_workspace_bytes -- bytes of device workspace a decode call needs:
 * per (sequence, KV head, query row, split) one fp32 max logit, one fp32
 * normalizer and head_dim fp32 partial outputs.  0 on invalid arguments.
 */
size_t kvq_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                           int32_t q_tokens, int32_t max_seq_len);

/*
 * kvq_decode_attend -- decode attention over a contiguous cache
 * (num_blocks = batch, block_size = capacity): kvq_split_decode followed by
 * kvq_combine.
 *
 *   q           bf16 [batch, q_tokens, num_q_heads, head_dim]
 *   seq_lens    int32 [batch] (device): cached tokens of each sequence,
 *               INCLUDING the q_tokens query tokens, which are the last ones.
 *               Query j sits at position seq_lens[b] - q_tokens + j and sees the
 *               tokens at or before it (causal among speculative drafts, [F]
 *               int4 XQA speculative decode).  A value above max_seq_len is
 *               treated as max_seq_len by every entry point, for reading and
 *               (fused append, prefill) for writing alike; 0 or less gives a
 *               zero output.
 *   max_seq_len host upper bound on seq_lens, <= the capacity; sizes the grid.
 *   softmax_scale logits are softmax_scale * q . k (usually 1/sqrt(head_dim)).
 *   head_sink   fp32 [num_q_heads] or NULL: per-head sink logit in post-scale
 *               units; the output of head h is multiplied by
 *               1 / (1 + exp(head_sink[h] - lse)) ([P] "CUDA kernels",
 *               ApplyHeadSink).
 *   out         bf16 [batch, q_tokens, num_q_heads, head_dim]
 *   workspace   device scratch of at least kvq_workspace_bytes(...) bytes.
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) ([K] "Method":
 * all query heads sharing a KV head are served from one read of it).  The
 * result is bitwise reproducible for a fixed shape and max_seq_len: the
 * splits merge in a fixed order and no atomics are used ([K] "Correctness").
 */
int kvq_decode_attend(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                      int32_t q_tokens, const int32_t* seq_lens, int32_t max_seq_len,
                      float softmax_scale, const float* head_sink, void* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * kvq_paged_decode_attend -- as kvq_decode_attend over a block-paged cache
 * ([P] "CUDA kernels": split-KV, block-table-aware paged decode).
 *   block_table int32 [batch, max_blocks]; max_seq_len <= max_blocks * block_size.
 * Entries outside [0, num_blocks) are a caller error; the kernel never reads
 * outside the pool and treats the tokens of such a block as absent.
 */
int kvq_paged_decode_attend(const kvq_cache* cache, const void* q, int32_t batch,
                            int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                            int32_t max_seq_len, float softmax_scale, const float* head_sink,
                            const int32_t* block_table, int32_t max_blocks, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_append_decode_attend -- one decode step in one call: quantize the query
 * tokens' new K and V rows into the cache, then attend ([P] "CUDA kernels":
 * the operator quantizes the new rows on write with ReshapeAndCache and then
 * runs the paged decode; [K] "Usage": append(k, v) followed by attend(q)).
 *
 *   k_new, v_new  bf16 [batch, q_tokens, num_kv_heads, head_dim]: row j of
 *                 sequence b is written at position L_b - q_tokens + j, with
 *                 L_b = min(seq_lens[b], max_seq_len) (the query tokens are the
 *                 last tokens of the sequence); rows before position 0 are not
 *                 written.
 *   block_table   int32 [batch, max_blocks], or NULL for the contiguous cache.
 *   Everything else as kvq_decode_attend / kvq_paged_decode_attend.
 *
 * The cache afterwards holds exactly what kvq_append(k_new, v_new,
 * positions = min(seq_lens, max_seq_len) - q_tokens) would have written, and
 * `out` equals that append followed by the decode.  The new rows are quantized inside the decode
 * kernel by the wavefront that reads them, which saves a launch per step.
 */
int kvq_append_decode_attend(const kvq_cache* cache, const void* k_new, const void* v_new,
                             const void* q, int32_t batch, int32_t num_q_heads, int32_t q_tokens,
                             const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                             const float* head_sink, const int32_t* block_table,
                             int32_t max_blocks, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * kvq_attend_ex -- the decode step with every option: an optional fused append
 * (k_new and v_new both non-NULL: as kvq_append_decode_attend; both NULL: the
 * cache already holds the rows), contiguous (block_table NULL) or paged cache,
 * optional head sink, and the attention options above (options NULL: none).
 * Arguments otherwise as kvq_append_decode_attend.  KVQ_EINVAL also for a
 * negative or non-finite soft cap, a negative window, or only one of k_new /
 * v_new.
 */
int kvq_attend_ex(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                  int32_t batch, int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                  int32_t max_seq_len, float softmax_scale, const float* head_sink,
                  const int32_t* block_table, int32_t max_blocks, const kvq_attn_options* options,
                  void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_attend_ex_noalloc -- kvq_attend_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, whose
 * place takes a scratch array of KVQ_NOALLOC_SCRATCH_BYTES that the library
 * holds in device memory (one per GPU, kept until the process ends).  The
 * call allocates nothing and computes exactly what kvq_attend_ex computes.
 *
 * Limit: a shape whose kvq_workspace_bytes exceeds KVQ_NOALLOC_SCRATCH_BYTES
 * returns KVQ_ESCRATCH before anything is enqueued (use kvq_attend_ex with a
 * caller workspace then).  Every call on one GPU uses that GPU's one array:
 * calls that overlap on a GPU (two streams, or two host threads, without an
 * order between them) race and give undefined results; calls ordered on one
 * stream are safe.  No content of the array carries from one call to the
 * next.  The first call whose stream belongs to a device looks up the
 * array's address on that device (a host query, no allocation); KVQ_EHIP if
 * the runtime refuses it.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int kvq_attend_ex_noalloc(const kvq_cache* cache, const void* k_new, const void* v_new,
                          const void* q, int32_t batch, int32_t num_q_heads, int32_t q_tokens,
                          const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                          const float* head_sink, const int32_t* block_table, int32_t max_blocks,
                          const kvq_attn_options* options, void* out, void* stream);

/*
 * The two phases the decode entry points are made of, for callers that
 * schedule them separately ([K] "Method": the sequence is split across
 * workgroups and the partials are merged in a fixed order).
 *
 * kvq_split_decode writes, for every chunk of every sequence, KV head and
 * query row, the chunk's max logit m, normalizer l and normalized partial
 * output into the workspace.  Chunks are cut over the whole batch: the T
 * 16-token tiles of all sequences are divided into chunks of
 * C = max(ceil(T / W), 8) tiles that never straddle two sequences
 * (W = kvq_num_splits), so ragged batches keep every workgroup equally busy.
 * block_table may be NULL (contiguous cache; max_blocks ignored).
 */
int kvq_split_decode(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                     int32_t q_tokens, const int32_t* seq_lens, int32_t max_seq_len,
                     float softmax_scale, const int32_t* block_table, int32_t max_blocks,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_combine merges the chunks of a preceding kvq_split_decode (same cache,
 * shape, seq_lens and max_seq_len) in chunk order, applies the static V scale
 * (per-tensor / per-channel), then the head sink, and writes bf16 `out`.
 * seq_lens (device) locates each sequence's chunks exactly as the split did.
 */
int kvq_combine(const kvq_cache* cache, int32_t batch, int32_t num_q_heads, int32_t q_tokens,
                const int32_t* seq_lens, int32_t max_seq_len, const float* head_sink, void* out,
                const void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_prefill_attend -- chunked prefill: q_tokens new tokens per sequence (a
 * prompt chunk) are quantized into the cache and attend causally to every
 * cached token up to their own ([K] "Requirements and limits": prefill runs a
 * tiled attention kernel, its keys and values go through the append; [F]
 * "Testing": prefill and chunked prefill over the paged quantized cache).
 *
 *   k_new, v_new  bf16 [batch, q_tokens, num_kv_heads, head_dim], both or
 *                 neither: written first, like kvq_append, at positions
 *                 min(seq_lens[b], max_seq_len) - q_tokens + j; NULL when the
 *                 chunk is already in the cache
 *   q             bf16 [batch, q_tokens, num_q_heads, head_dim]
 *   seq_lens      int32 [batch] (device): tokens of each sequence after the
 *                 chunk; a value above max_seq_len is treated as max_seq_len
 *   out           bf16 [batch, q_tokens, num_q_heads, head_dim]
 *   options       soft cap / sliding window as kvq_attend_ex, or NULL
 *   Everything else as kvq_attend_ex.  Query token j of sequence b sits at
 *   position seq_lens[b] - q_tokens + j and attends every cached token at or
 *   before it (inside the window); the output is exact softmax attention over
 *   the dequantized cache, like the decode, so a chunk of one token is a
 *   decode step.  Tokens before position 0 output zeros.  q_tokens has no
 *   upper bound beyond G * q_tokens < 2^30; no workspace is needed (one
 *   workgroup owns 64 or 128 query rows of one KV head over all its tokens).
 *   Two launches on `stream` (append, attention); graph-capturable.
 */
int kvq_prefill_attend(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                       int32_t batch, int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                       int32_t max_seq_len, float softmax_scale, const float* head_sink,
                       const int32_t* block_table, int32_t max_blocks,
                       const kvq_attn_options* options, void* out, void* stream);

/*
 * kvq_prefill_workspace_bytes -- device workspace for kvq_prefill_attend_ws:
 * when the prefill's workgroups (one per 64 or 128 query rows of a KV head)
 * would leave part of the GPU idle in their last round, each one's cached
 * tiles are cut into up to 8 consecutive parts of one workgroup each, whose
 * partial outputs the workspace holds until a fixed-order merge ([K]
 * "Method": the sequence is split across workgroups and the partials are
 * merged in a fixed order).  A host-only, pure function of the shape
 * (options: its sliding window, or NULL); 0 when no split pays, or for an
 * invalid shape.  Holds batch * num_kv_heads * G * q_tokens * parts rows of
 * head_dim + 2 floats.
 */
size_t kvq_prefill_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                   int32_t q_tokens, int32_t max_seq_len,
                                   const kvq_attn_options* options);

/*
 * kvq_prefill_attend_ws -- kvq_prefill_attend with that workspace: the same
 * arguments and result (up to the rounding of the merge), with the split.
 * workspace (device, 16-byte aligned) must hold kvq_prefill_workspace_bytes
 * for the same shape and options (it may be NULL when that is 0), else
 * KVQ_EINVAL before anything is enqueued; the caller owns it, and calls that
 * overlap must not share it.  Up to three launches on `stream` (append,
 * attention, merge); graph-capturable.
 */
int kvq_prefill_attend_ws(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                          int32_t batch, int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                          int32_t max_seq_len, float softmax_scale, const float* head_sink,
                          const int32_t* block_table, int32_t max_blocks,
                          const kvq_attn_options* options, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * kvq_cache_bytes -- host-only footprint of one layer's cache: codes of K and
 * V plus, for KVQ_PER_ROW, one fp32 scale per row ([K] opening paragraphs
 * and "Cache footprint"; [F] "Motivation and Context": static per-channel
 * scales add nothing per token).  Static tables are not counted.  KVQ_BF16
 * (with KVQ_NO_SCALE) counts 2 * head_dim bytes per row.
 */
size_t kvq_cache_bytes(int32_t dtype, int32_t scale_mode, int32_t num_kv_heads, int32_t head_dim,
                       int64_t tokens);

/* Human-readable name of a kvq_status (host, static storage). */
const char* kvq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
