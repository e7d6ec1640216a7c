/*
 * sfa.h -- C ABI of libsfa.so: sparse flash attention (SFA) over a paged MLA latent KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation ("DeepSeek V3/V2 Sparse Flash Attention with Quantization", sections
 * "Algorithm overview", "Operator specification", "Input/output parameters";
 * "CANN DeepSeek Indexer attention optimisation", section "Sparse Flash Attention"):
 *
 *   For query token t = b*s1 + s and head h, each slot k of topk_indices[t] names a logical
 *   position j of batch b's cache. Slot k is valid iff 0 <= j < kv_act_seqs[b]. A valid slot
 *   reads physical row  row = block_table[b][j / 128] * 128 + j % 128.
 *   Then
 *     score[k] = softmax_scale * ( q_nope[t,h] . Kn[row] + q_rope[t,h] . Kr[row] )
 *     out[b,s,h,:] = sum over valid k of softmax_k(score)[k] * Kn[row_k]      (V = k_nope)
 *   Kn is key_nope_2d. With an INT8 cache it is the dequantised value: the int8 code becomes
 *   fp32 exactly, is multiplied in fp32 by the scale of its 128-element group, and the product
 *   is rounded to bf16. The output is rounded to bf16 (round to nearest even).
 *   A token with no valid slot outputs zeros. Invalid slots may sit anywhere in the row.
 *
 * Conventions common to every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous row-major buffers. The caller owns
 *     them and keeps them alive until the work queued on `stream` has finished. The library
 *     never allocates, frees, or keeps a pointer after it returns.
 *   - Calls are asynchronous: the library only queues kernels on `stream` and never
 *     synchronises. A fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Return value: SFA_OK (0), or a negative sfa_status. Argument errors are found by
 *     synchronous host-side validation before anything is queued; in that case nothing runs
 *     and `out` is untouched. SFA_ERR_HIP means a HIP call failed (see sfa_status_string).
 *   - Data preconditions, not checked on the host:
 *       * every block_table entry that a valid slot reaches lies in
 *         [0, num_cache_rows / 128);
 *       * kv_act_seqs[b] <= max_blocks_per_batch * 128.
 *     The kernels never dereference a row outside [0, num_cache_rows), nor a block_table
 *     column at or past max_blocks_per_batch. Slots that would need one are treated as
 *     masked.
 *   - Entry points are reentrant. Calls on different streams may overlap if they use
 *     different output and workspace buffers.
 */
#ifndef SFA_H_
#define SFA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFA_KV_LORA_RANK 512  /* nope width: query_nope, key_nope_2d, attention_out columns */
#define SFA_ROPE_DIM 64       /* rope width: query_rope, key_rope_2d columns                 */
#define SFA_BLOCK_SIZE 128    /* cache rows per page                                        */
#define SFA_QUANT_GROUP 128   /* INT8 elements sharing one FP32 scale (4 scales per row)     */
#define SFA_MAX_HEADS 128     /* query heads sharing the single latent KV head               */

typedef enum { SFA_KV_BF16 = 0, SFA_KV_INT8 = 1 } sfa_kv_dtype;

typedef enum {
  SFA_OK = 0,
  SFA_ERR_NULL = -1,            /* a required pointer is NULL                                 */
  SFA_ERR_DIMS = -2,            /* a dimension is outside what the library supports           */
  SFA_ERR_ALIGN = -3,           /* a tensor pointer is not 16-byte aligned                    */
  SFA_ERR_WORKSPACE = -4,       /* workspace missing, misaligned, or smaller than required    */
  SFA_ERR_SCALES = -5,          /* INT8 cache without k_nope_scales                           */
  SFA_ERR_ALIAS = -6,           /* an output overlaps an input or the workspace, or the
                                   workspace overlaps an input                                */
  SFA_ERR_SCALE_VALUE = -7,     /* softmax_scale is not finite                                */
  SFA_ERR_HIP = -8,             /* a HIP runtime call failed                                  */
  SFA_ERR_SCRATCH_LIMIT = -9    /* sfa_decode_noalloc: the call needs more than its fixed
                                   scratch (SFA_NOALLOC_SCRATCH_BYTES)                         */
} sfa_status;

/* Shapes of one call ("Input/output parameters" table of the SFA-with-quantisation page).
 * T = batch * s1 query tokens. */
typedef struct {
  int32_t batch;                /* B >= 0                                                     */
  int32_t s1;                   /* query tokens per batch >= 0 (decode: 1 or 2; prefill: many) */
  int32_t n_q;                  /* query heads: a multiple of 16 in [16, 128]                 */
  int32_t n_kv;                 /* latent KV heads: must be 1                                 */
  int32_t kv_lora_rank;         /* must be 512                                                */
  int32_t rope_dim;             /* must be 64                                                 */
  int32_t block_size;           /* must be 128                                                */
  int32_t topk;                 /* slots per token (row length of topk_indices), >= 1         */
  int32_t max_blocks_per_batch; /* row length of block_table, >= 1                            */
  int64_t num_cache_rows;       /* block_num * block_size: rows of key_nope_2d / key_rope_2d  */
  sfa_kv_dtype kv_dtype;        /* SFA_KV_INT8 => k_nope_scales is required                   */
  int32_t num_splits;           /* 0 = automatic. Otherwise the number of top-k partitions per
                                   token (raised to ceil(topk/2048) when smaller). Used only for
                                   tests and tuning; every value gives the same result within
                                   the accuracy standard. */
} sfa_dims;

/*
 * Bytes of device workspace that sfa_decode (is_prefill = 0) or sfa_prefill (is_prefill = 1)
 * needs for `dims`. Host-only: no GPU is touched. *bytes_out may be 0, in which case the
 * workspace pointer may be NULL.
 *
 * The workspace holds per-partition partial results and 82 64-bit counter words per token
 * (partitions arrived, partials published, and the flags of the spread merge, in which each of
 * 2 to 16 partitions merges a share of the output). It needs no initialisation: every call tags
 * its counters with a 48-bit generation of its own, so whatever the buffer held before counts
 * as zero. The environment variable SFA_MERGE_WAIT_NS bounds, in nanoseconds, how long an early
 * partition waits for the others' partials before leaving its share to the last (default
 * 50,000; 0 turns the spread merge off): the result is the same either way.
 */
int sfa_workspace_size(const sfa_dims* dims, int is_prefill, size_t* bytes_out);

/*
 * Decode-mode SFA ("Decode mode": s1 of 1 or 2, standard softmax over the token's top-k set).
 *
 *   query_nope     bf16  (T*n_q, 512)      row (b*s1 + s)*n_q + h
 *   query_rope     bf16  (T*n_q, 64)
 *   key_nope_2d    bf16 or int8 (num_cache_rows, 512)
 *   key_rope_2d    bf16  (num_cache_rows, 64)
 *   k_nope_scales  fp32  (num_cache_rows, 4)  INT8 only (NULL allowed for bf16)
 *   topk_indices   int32 (T, topk)           logical positions, -1 = padding
 *   block_table    int32 (batch, max_blocks_per_batch)
 *   kv_act_seqs    int32 (batch)
 *   softmax_scale  multiplies the raw score before the softmax (finite)
 *   out            bf16  (batch, s1, n_q, 512)   written in full
 *   workspace      device buffer of >= sfa_workspace_size(dims, 0) bytes, 256-byte aligned,
 *                  contents need not be initialised (see above)
 * Every tensor pointer must be 16-byte aligned.
 *
 * The top-k set of each token is split into partitions that run in parallel, each with an
 * online (running max / running sum) softmax over 32-slot tiles. The partials are merged with
 * the log-sum-exp law in the same kernel: the prefill mode's update rule applied across
 * partitions.
 */
int sfa_decode(const sfa_dims* dims,
               const void* query_nope, const void* query_rope,
               const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
               const int32_t* topk_indices, const int32_t* block_table, const int32_t* kv_act_seqs,
               float softmax_scale, void* out,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sfa_decode without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, layouts, results and errors are those of sfa_decode. The workspace that
 * sfa_decode would take is instead a fixed array inside this library, SFA_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, held by every GPU the library runs on until the process ends. Its device
 * address is looked up on the first call on each device. The call allocates and frees nothing.
 *   - A call whose sfa_workspace_size(dims, 0) exceeds SFA_NOALLOC_SCRATCH_BYTES returns
 *     SFA_ERR_SCRATCH_LIMIT and queues nothing; a smaller dims.num_splits needs less.
 *     The limit covers decode of 64 sequences x 2 query tokens x top-k 2048 with the automatic
 *     partition choice (256 partitions of 256 KB each).
 *   - Every call on one GPU shares that GPU's array: calls that may overlap on one GPU (on
 *     different streams, or from different threads) race and give wrong results. Calls queued
 *     on one stream are ordered and safe. The array keeps the last call's contents; nothing
 *     in it needs clearing, since each call tags its counters with a generation of its own.
 */
#define SFA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
int sfa_decode_noalloc(const sfa_dims* dims,
                       const void* query_nope, const void* query_rope,
                       const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
                       const int32_t* topk_indices, const int32_t* block_table, const int32_t* kv_act_seqs,
                       float softmax_scale, void* out, hipStream_t stream);

/*
 * Prefill-mode SFA ("Prefill mode": many query tokens; an online softmax keeps the running
 * output, running sum and running max across s2 tiles and normalises at the last tile).
 * Same arguments and layouts as sfa_decode. Each token runs in one workgroup, with no
 * partitioning while topk <= 2048, and tokens are scheduled latest-first. In causal prefill
 * the later tokens hold the most valid slots, so they start first.
 */
int sfa_prefill(const sfa_dims* dims,
                const void* query_nope, const void* query_rope,
                const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
                const int32_t* topk_indices, const int32_t* block_table, const int32_t* kv_act_seqs,
                float softmax_scale, void* out,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The gather step alone: rows_out (T, topk) int32 receives the physical cache row of every
 * valid slot and -1 for every masked one (PagedAttention mapping, blocks of 128 rows). It
 * exposes the index resolution that sfa_decode / sfa_prefill perform internally, so that it
 * can be checked bit-exactly.
 */
int sfa_resolve_rows(const sfa_dims* dims, const int32_t* topk_indices, const int32_t* block_table,
                     const int32_t* kv_act_seqs, int32_t* rows_out, hipStream_t stream);

/*
 * ---- Cache write: the step that fills the latent cache ----
 *
 * "DeepSeek V3/V2 Sparse Flash Attention with Quantization", sections "Algorithm overview"
 * (PagedAttention) and "INT8 quantisation rule". New token t = b*s1 + s carries one latent row
 * (512 nope + 64 rope, bf16) for logical position p = positions[t] of batch b; it is written at
 * physical row block_table[b][p / 128] * 128 + p % 128 of the cache that sfa_decode and
 * sfa_prefill read.
 *   BF16 cache: nope and rope are copied bit for bit.
 *   INT8 cache: rope is copied; each 128-element group of nope is quantised as
 *     scale = absmax(group) / 127             (fp32, IEEE division, round to nearest even)
 *     code  = clamp(round_half_even(x / scale), -128, 127)   (x / scale one fp32 division)
 *   and an all-zero group stores scale 0 and codes 0. The attention's dequant chain then reads
 *   code * scale rounded to bf16.
 *
 *   dims           batch, s1, kv_lora_rank (512), rope_dim (64, or 0), block_size (128),
 *                  max_blocks_per_batch, num_cache_rows and kv_dtype are used; n_q, n_kv, topk
 *                  and num_splits are ignored. T = batch * s1 may be up to 2^26. rope_dim 0 is
 *                  the 512-wide row layout sfa_window_decode reads with rope_dim 0 (rotary
 *                  channels inside the row): there is no rope part, the 512 channels are new_nope
 *                  (quantised whole for an INT8 cache), and new_rope and key_rope_2d are not used
 *                  (they may be NULL).
 *   new_nope       bf16  (T, 512)
 *   new_rope       bf16  (T, 64)
 *   positions      int32 (T)
 *   block_table    int32 (batch, max_blocks_per_batch)
 *   key_nope_2d    bf16 or int8 (num_cache_rows, 512)   written in place
 *   key_rope_2d    bf16  (num_cache_rows, 64)           written in place
 *   k_nope_scales  fp32  (num_cache_rows, 4)            written in place; INT8 only (NULL for bf16)
 *
 * A token is not written when p < 0, p >= max_blocks_per_batch * 128, its block_table entry is
 * negative, or its row is outside [0, num_cache_rows). Rows no token targets are untouched.
 * Preconditions, not checked: no two written tokens target the same row (which of them lands is
 * otherwise unspecified); the nope values are finite. Errors: SFA_ERR_NULL, SFA_ERR_DIMS,
 * SFA_ERR_SCALES (INT8 without scales), SFA_ERR_ALIGN (any pointer not 16-byte aligned),
 * SFA_ERR_ALIAS (an output overlaps an input or another output), SFA_ERR_HIP. Asynchronous on
 * `stream`, no allocation, like every entry point.
 */
int sfa_cache_write(const sfa_dims* dims, const void* new_nope, const void* new_rope, const int32_t* positions,
                    const int32_t* block_table, void* key_nope_2d, void* key_rope_2d, float* k_nope_scales,
                    hipStream_t stream);

/*
 * ---- Sliding-window + compressed-cache attention: SWA, CFA and SCFA ----
 *
 * "NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section "FA-class operators: SWA,
 * CFA and SCFA": a query reads a sliding window of the original cache (ori_kv) and, for CFA and
 * SCFA, entries of the compressed cache (cmp_kv): every causal one (CFA) or those a sparse
 * index list selects (SCFA). SWA has the window alone. The attention over the union of the two
 * row sets is the one of sfa_decode (same scores, softmax, V = nope, accuracy and output).
 *
 *   Query token t = b*s1 + s sits at position p = ori_len[b] - s1 + s. Its rows are
 *     - the original-cache positions max(0, p - window + 1) .. p, through block_table_ori;
 *     - cmp_indices[t, i] for i < topk_cmp, valid iff 0 <= c < cmp_len[b], through
 *       block_table_cmp (-1 or out-of-range entries are masked anywhere in the row; for CFA the
 *       caller lists every causal entry, for SCFA the selected ones).
 *   Both caches are rows of one paged pool (key_nope_2d, key_rope_2d, k_nope_scales as in
 *   sfa_decode, blocks of 128 rows); each has its own block table and length.
 *
 *   rope_dim 64: rows and queries of 512 nope + 64 rope channels, as in sfa_decode.
 *   rope_dim 0: the page's D = 512 layout (the head size its timing table gives these
 *     operators): 512-channel rows whose last 64 channels already carry the rotary embedding
 *     (applied in place by the prolog or the compressor). The score is q . k over the 512
 *     channels and V is the same row; query_rope and key_rope are not read and may be NULL.
 *     An INT8 pool holds the whole row as codes, with 4 group scales per row as in sfa_decode.
 *
 *   query_nope/query_rope/out/key_*    as for sfa_decode
 *   cmp_indices      int32 (T, topk_cmp)                    NULL when topk_cmp == 0
 *   block_table_ori  int32 (batch, max_blocks_ori)
 *   block_table_cmp  int32 (batch, max_blocks_cmp)          NULL when topk_cmp == 0
 *   ori_len, cmp_len int32 (batch)                          cmp_len NULL when topk_cmp == 0
 *   workspace        as for sfa_decode, sized by sfa_window_workspace_size (0 bytes, and NULL
 *                    allowed, when the slots need no partitions)
 *
 * The window and the compressed list form the slot list of the sparse attention kernel: the
 * kernel resolves both in its own prologue (original positions through block_table_ori,
 * compressed entries through block_table_cmp) and runs unchanged after it. Queued on `stream`;
 * nothing is allocated. Errors as for sfa_decode, plus SFA_ERR_DIMS for window < 0,
 * topk_cmp < 0, window + topk_cmp < 1 (or above the attention's top-k limit),
 * max_blocks_ori < 1, topk_cmp > 0 with max_blocks_cmp < 1, or rope_dim other than 64 or 0.
 * Preconditions as for sfa_decode, on both block tables; also ori_len[b] >= s1 for a full window
 * (positions below 0 are simply absent).
 */
typedef struct {
  int32_t batch, s1, n_q, n_kv, kv_lora_rank, rope_dim, block_size;  /* as in sfa_dims, but
                                                                        rope_dim 64 or 0      */
  int32_t window;          /* original-cache positions each query reads, >= 0               */
  int32_t topk_cmp;        /* row length of cmp_indices, >= 0 (0: SWA, no compressed source)  */
  int32_t max_blocks_ori;  /* row length of block_table_ori, >= 1                            */
  int32_t max_blocks_cmp;  /* row length of block_table_cmp (>= 1 when topk_cmp > 0)         */
  int64_t num_cache_rows;  /* rows of the shared pool                                        */
  sfa_kv_dtype kv_dtype;
  int32_t num_splits;      /* as in sfa_dims (0 = automatic)                                 */
} sfa_window_dims;

int sfa_window_workspace_size(const sfa_window_dims* dims, size_t* bytes_out);
int sfa_window_decode(const sfa_window_dims* dims, const void* query_nope, const void* query_rope,
                      const void* key_nope_2d, const void* key_rope_2d, const float* k_nope_scales,
                      const int32_t* cmp_indices, const int32_t* block_table_ori, const int32_t* block_table_cmp,
                      const int32_t* ori_len, const int32_t* cmp_len, float softmax_scale, void* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char* sfa_status_string(int status);

/* Number of top-k partitions per token that sfa_decode (is_prefill = 0) or sfa_prefill
 * (is_prefill = 1) will use for `dims` (host-only). Returns a negative sfa_status on bad dims. */
int sfa_num_splits(const sfa_dims* dims, int is_prefill);

/*
 * ---- Lightning Indexer and top-k selection: the step that produces topk_indices ----
 *
 * "CANN DeepSeek Indexer attention optimisation", sections "Lightning Indexer" and "Sparse
 * Flash Attention": for query token i and cache position j the index score is
 *     I[i, j] = sum over index heads h of w[i, h] * ReLU(q_index[i, h] . k_index[j]),
 * and token i attends to the k positions with the largest I[i, :]. The index keys live in a
 * paged cache with the same block table and live lengths as the latent cache (the operator's
 * prototype passes index_k_cache beside block_table and act_seqs).
 *
 * The conventions of the attention entry points hold: device pointers, 16-byte alignment,
 * asynchronous on `stream`, synchronous host validation with the same status codes, no
 * allocation. Position j of batch b is live iff 0 <= j < kv_act_seqs[b] (both tokens of an
 * MTP pair share the bound); the same data preconditions on block_table apply.
 */
typedef struct {
  int32_t batch;
  int32_t s1;                   /* query tokens per batch; T = batch * s1                       */
  int32_t n_heads;              /* index heads: must be 64                                      */
  int32_t head_dim;             /* index head dim: must be 128                                  */
  int32_t block_size;           /* must be 128                                                  */
  int32_t max_blocks_per_batch; /* row length of block_table; positions per token = 128 * this  */
  int64_t num_cache_rows;       /* rows of index_k_cache                                        */
  int32_t topk;                 /* positions selected per token (>= 1)                          */
} sfa_indexer_dims;

/*
 * Index scores.
 *   q_index        bf16  (T*64, 128)    row t*64 + h
 *   k_index_cache  bf16  (num_cache_rows, 128)
 *   weights        fp32  (T, 64)        the per-token head weights w[i, :]
 *   block_table    int32 (batch, max_blocks_per_batch)
 *   kv_act_seqs    int32 (batch)
 *   scores         fp32  (T, max_blocks_per_batch*128), written in full: I[t, j] for live j,
 *                  -inf for every other position
 * Dot products accumulate in fp32 from exact bf16 products; ReLU, weighting and the head sum
 * are fp32.
 */
int sfa_indexer_scores(const sfa_indexer_dims* dims, const void* q_index, const void* k_index_cache,
                       const float* weights, const int32_t* block_table, const int32_t* kv_act_seqs,
                       float* scores, hipStream_t stream);

/*
 * Top-k selection over the scores of sfa_indexer_scores (same dims and kv_act_seqs).
 *   topk_indices   int32 (T, topk)  output: the logical positions of the topk largest scores
 *                  of each token's live positions, in no particular order. With fewer live
 *                  positions than topk, all of them are selected (in position order) and the
 *                  rest of the row is -1. The result can be passed straight to sfa_decode.
 * Among scores equal to the k-th largest, the lowest positions are taken (-0.0 equals +0.0).
 * The selection is exact on the fp32 scores given. A NaN score ranks by its sign bit: above
 * +inf when positive, below -inf when negative (sfa_indexer_scores never writes one).
 */
int sfa_topk_select(const sfa_indexer_dims* dims, const float* scores, const int32_t* kv_act_seqs,
                    int32_t* topk_indices, hipStream_t stream);

/*
 * ---- Compressor: the step that fills the compressed cache the window attention reads ----
 *
 * "NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section "Compressor", its
 * computation steps. The two projections of the new tokens' hidden states (plain GEMMs, done
 * by the caller) arrive as kv and score. Token t = b*s1 + s at position p = start_pos[b] + s,
 * taken in order of s, refreshes slot p % ratio of its sequence's state:
 *     kv_state[b][slot] = kv[t]        score_state[b][slot] = score[t] + ape[slot]   (fp32 add)
 * When p + 1 is a multiple of ratio, the state is pooled into compressed entry
 * c = (p + 1) / ratio - 1:
 *     x[ch] = sum over slots r of softmax_r(score_state[b][r][ch]) * kv_state[b][r][ch]
 *     y     = x / sqrt(mean over the C channels of x^2 + eps) * gamma
 *     y[C - 64 + 2i], y[C - 63 + 2i]  rotated by the angle with cosine rope_cos[p][i] and sine
 *                                     rope_sin[p][i] (i < 32; adjacent pairs)
 * With rotate = 1 (128 channels only) y then becomes H y / sqrt(128), H the Sylvester Hadamard
 * matrix in natural order (H_2n = [[H_n, H_n], [H_n, -H_n]]), the page's rotate = true branch.
 * y is stored as bf16 (round to nearest even) at row block_table_cmp[b][c / 128] * 128 + c % 128:
 * with 576 channels, channels 0..511 to key_nope_2d and 512..575 to key_rope_2d (the row layout
 * of the cache sfa_window_decode reads with rope_dim 64); with 512 channels (the page's D = 512
 * layout, the row sfa_window_decode reads with rope_dim 0) or 128 channels (the page's D = 128
 * configuration, an index-key row for the Lightning Indexer), the whole row to key_nope_2d
 * (key_rope_2d is not used and may be NULL). The softmax, sum, norm and rotations are fp32.
 *
 *   dims              channels C = 576, 512 or 128, rotate 0 or 1 (1 only with 128), block_size
 *                     128; ratio in [1, 1024]; T = batch*s1 up to 2^26; max_blocks = row
 *                     length of block_table_cmp
 *   kv, score         fp32  (T, C)
 *   ape               fp32  (ratio, C)        added to the score of the slot it is indexed by
 *   gamma             fp32  (C)
 *   eps               finite, >= 0
 *   rope_cos/sin      fp32  (rope_positions, 32)
 *   start_pos         int32 (batch)
 *   kv_state,
 *   score_state       fp32  (batch, ratio, C), read and refreshed in place
 *   block_table_cmp   int32 (batch, max_blocks)
 *   key_nope_2d       bf16  (num_cache_rows, 512) for C = 576 or 512, or (num_cache_rows, 128)
 *                     for C = 128, written in place
 *   key_rope_2d       bf16  (num_cache_rows, 64) written in place (C = 576 only)
 *
 * With batch * s1 = 0 the call reads nothing and returns SFA_OK (the pointers may then be NULL).
 * A token with p < 0 or p >= rope_positions is skipped (no refresh, no entry). An entry is not
 * written when c >= max_blocks * 128, its block entry is negative, or its row is outside
 * [0, num_cache_rows); the state is still refreshed. Precondition, not checked: the inputs are
 * finite. Errors: SFA_ERR_NULL, SFA_ERR_DIMS, SFA_ERR_ALIGN (any pointer not 16-byte aligned),
 * SFA_ERR_ALIAS (an output overlaps an input or another output), SFA_ERR_HIP. Asynchronous on
 * `stream`, no allocation.
 */
typedef struct {
  int32_t batch;
  int32_t s1;                   /* new tokens per sequence                                      */
  int32_t channels;             /* 576 (kv_lora_rank + rope_dim), 512 (rotary channels inside the
                                   row) or 128 (an index-key row)                                */
  int32_t ratio;                /* compression ratio                                            */
  int32_t rope_positions;       /* rows of rope_cos and rope_sin                                */
  int32_t max_blocks;           /* row length of block_table_cmp                                */
  int32_t block_size;           /* must be 128                                                  */
  int32_t rotate;               /* 0, or 1: the Hadamard transform after RoPE (128 channels)    */
  int64_t num_cache_rows;       /* rows of the compressed pool                                  */
} sfa_compress_dims;

int sfa_compress(const sfa_compress_dims* dims, const float* kv, const float* score, const float* ape,
                 const float* gamma, float eps, const float* rope_cos, const float* rope_sin,
                 const int32_t* start_pos, float* kv_state, float* score_state, const int32_t* block_table_cmp,
                 void* key_nope_2d, void* key_rope_2d, hipStream_t stream);

/*
 * MLA prolog: the new tokens' hidden states to the absorbed query that sfa_decode reads and the
 * latent row that sfa_cache_write stores ("CANN DeepSeek Indexer attention optimisation",
 * section "MLA Prolog" and the prolog's parameter list: DeepSeek V3's structure with weight
 * absorption in decode; "NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section
 * "MlaProlog", computation steps: down-projection, RMSNorm, up-projection, interleaved RoPE on
 * the last rope_dim channels; the key a projection, RMSNorm, RoPE). For token t with hidden row
 * x and position p = positions[t]:
 *
 *   cq         = RMSNorm(x . w_dq^T) * gamma_cq                              (Q channels)
 *   u          = cq . w_uq_qr^T; head h: qn = u[h*(Dn+64) + 0 .. Dn), qp = u[h*(Dn+64) + Dn .. +64)
 *   q_nope[t,h] = qn . w_uk[h]^T                                             (512 channels)
 *   q_rope[t,h] = RoPE(qp, p)
 *   kv         = x . w_dkv_kr^T; kv_nope[t] = RMSNorm(kv[0..512)) * gamma_ckv; kv_rope[t] = RoPE(kv[512..576), p)
 *
 * RMSNorm(v) = v / sqrt(mean(v^2) + eps). RoPE turns each adjacent pair (2i, 2i+1) by the angle
 * whose cosine and sine are rope_cos[p][i] and rope_sin[p][i]; a token with p outside
 * [0, rope_positions) gets zero q_rope and kv_rope. The products accumulate in fp32; cq and qn
 * are carried between the steps as bf16 hi + lo pairs (about 16 significant bits), not
 * rounded to bf16. The outputs are rounded to bf16 (nearest even).
 *
 *   x          bf16 (T, H)
 *   w_dq       bf16 (Q, H)              (out_features, in_features), as every weight here
 *   gamma_cq   bf16 (Q)
 *   w_uq_qr    bf16 (n_q*(Dn+64), Q)   head h owns rows h*(Dn+64) .. +Dn+64: nope, then rope
 *   w_uk       bf16 (n_q, 512, Dn)     w_uk[h][c][d] weighs qn[d] into q_nope[c]
 *   w_dkv_kr   bf16 (576, H)           rows 0..511 the latent row, 512..575 the rotary key
 *   gamma_ckv  bf16 (512)
 *   positions  int32 (T)
 *   rope_cos, rope_sin  fp32 (rope_positions, 32)
 *   q_nope     bf16 (T*n_q, 512)       row t*n_q + h: sfa_decode's query_nope
 *   q_rope     bf16 (T*n_q, 64)        sfa_decode's query_rope
 *   kv_nope    bf16 (T, 512), kv_rope bf16 (T, 64): sfa_cache_write's new_nope / new_rope
 *   cq_out     bf16 (T, Q), or NULL: cq rounded to bf16 (the indexer prolog's qr input)
 *   workspace  >= sfa_mla_prolog_workspace_size bytes, 256-byte aligned, no initialisation
 *
 * Errors: SFA_ERR_NULL, SFA_ERR_DIMS, SFA_ERR_ALIGN (any pointer not 16-byte aligned),
 * SFA_ERR_WORKSPACE, SFA_ERR_ALIAS (an output overlaps an input, another output or the
 * workspace), SFA_ERR_HIP. With T = 0 nothing is read or queued and the pointers may be NULL.
 * Asynchronous on `stream`, no allocation. Two calls that may overlap need separate
 * workspaces.
 */
typedef struct {
  int32_t tokens;               /* T >= 0 new tokens                                          */
  int32_t hidden;               /* H: a multiple of 64 in [64, 65536]                         */
  int32_t q_lora_rank;          /* Q: a multiple of 64 in [64, 4096]                          */
  int32_t n_q;                  /* query heads in [1, 128]                                    */
  int32_t qk_nope_dim;          /* Dn: per-head nope width before absorption, a multiple of 64
                                   in [64, 512]                                               */
  int32_t rope_positions;       /* rows of rope_cos and rope_sin, >= 1                        */
  float eps;                    /* RMSNorm epsilon, finite and >= 0                           */
} sfa_prolog_dims;

int sfa_mla_prolog_workspace_size(const sfa_prolog_dims* dims, size_t* bytes_out);
int sfa_mla_prolog(const sfa_prolog_dims* dims, const void* x, const void* w_dq, const void* gamma_cq,
                   const void* w_uq_qr, const void* w_uk, const void* w_dkv_kr, const void* gamma_ckv,
                   const int32_t* positions, const float* rope_cos, const float* rope_sin, void* q_nope,
                   void* q_rope, void* kv_nope, void* kv_rope, void* cq_out, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * MLA prolog, V4 form: the new tokens' hidden states to 512-wide query heads and a 512-wide
 * latent row, each with its rotary part inside ("NPU DeepSeek-V4 model PyPTO fused-operator
 * optimisation", section "MlaProlog", computation steps: two projections and RMSNorms for the
 * query, the second RMSNorm with its weight fixed at 1, one projection and RMSNorm for the key,
 * and interleaved RoPE in place on the last rope_dim channels of both). For token t with hidden
 * row x and position p = positions[t]:
 *
 *   cq      = RMSNorm(x . w_dq^T) * gamma_cq                      (Q channels)
 *   q[t,h]  = RMSNorm(cq . w_uq[h]^T), unit weight, over the head's 512 channels;
 *             then RoPE(p) in place on channels 448 .. 511
 *   kv[t]   = RMSNorm(x . w_dkv^T) * gamma_ckv over 512 channels; then RoPE(p) in place on
 *             channels 448 .. 511
 *
 * These are the rows sfa_window_decode reads with rope_dim 0 (query_nope) and sfa_cache_write
 * writes with rope_dim 0 (new_nope). RMSNorm and RoPE as for sfa_mla_prolog (a token with p
 * outside [0, rope_positions) gets zeros in its rotary channels); products accumulate in fp32, cq
 * is carried as a bf16 hi + lo pair into the up-projection, outputs are rounded to bf16.
 *
 *   x          bf16 (T, H)
 *   w_dq       bf16 (Q, H)              (out_features, in_features)
 *   gamma_cq   bf16 (Q)
 *   w_uq       bf16 (n_q*512, Q)        head h owns rows h*512 .. h*512 + 511
 *   w_dkv      bf16 (512, H)
 *   gamma_ckv  bf16 (512)
 *   positions  int32 (T); rope_cos, rope_sin fp32 (rope_positions, 32)
 *   q          bf16 (T*n_q, 512)        row t*n_q + h
 *   kv         bf16 (T, 512)
 *   cq_out     bf16 (T, Q), or NULL: cq rounded to bf16
 *   workspace  >= sfa_mla_prolog_v4_workspace_size bytes, 256-byte aligned, no initialisation
 *
 * Errors: SFA_ERR_NULL, SFA_ERR_DIMS (hidden and q_lora_rank multiples of 64 in [64, 65536] and
 * [64, 4096], n_q in [1, 128], head_dim 512, rope_positions >= 1, eps finite and >= 0, tokens up
 * to 2^20), SFA_ERR_ALIGN (16 bytes), SFA_ERR_ALIAS (an output overlapping an input, another
 * output or the workspace), SFA_ERR_WORKSPACE, SFA_ERR_HIP. With tokens = 0 nothing is read.
 * Asynchronous on `stream`, no allocation.
 */
typedef struct {
  int32_t tokens;               /* T >= 0 new tokens                                          */
  int32_t hidden;               /* H                                                          */
  int32_t q_lora_rank;          /* Q                                                          */
  int32_t n_q;                  /* query heads                                                */
  int32_t head_dim;             /* must be 512                                                */
  int32_t rope_positions;       /* rows of rope_cos and rope_sin, >= 1                        */
  float eps;                    /* RMSNorm epsilon                                            */
} sfa_prolog_v4_dims;

int sfa_mla_prolog_v4_workspace_size(const sfa_prolog_v4_dims* dims, size_t* bytes_out);
/* kv_ready: NULL, or an event that the call records on `stream` as soon as kv and cq_out are
 * complete, before the query up-projection (its longest launch): work that reads only kv or cq
 * (the cache write of kv, the Indexer Prolog on cq) can wait for it on another stream and run
 * beside the rest of the call. */
int sfa_mla_prolog_v4(const sfa_prolog_v4_dims* dims, const void* x, const void* w_dq, const void* gamma_cq,
                      const void* w_uq, const void* w_dkv, const void* gamma_ckv, const int32_t* positions,
                      const float* rope_cos, const float* rope_sin, void* q, void* kv, void* cq_out,
                      void* workspace, size_t workspace_bytes, hipEvent_t kv_ready, hipStream_t stream);

/*
 * Indexer prolog: the new tokens' inputs of the Lightning Indexer ("CANN DeepSeek Indexer
 * attention optimisation", section "Indexer Prolog": the index query RoPE(RMSNorm(X W_qa) W_qb),
 * the index key RoPE(LayerNorm(X W_k)), RoPE on the second half of the head dimension, the
 * head weights from a projection of x; "NPU DeepSeek-V4 model PyPTO fused-operator
 * optimisation", section "IndexerProlog": the Hadamard transform after RoPE and the weights'
 * 1/sqrt(heads * head_dim) scale). For token t with hidden row x, normalised query qr (the MLA
 * prolog's cq: sfa_mla_prolog's cq_out) and position p:
 *
 *   q[h]    = (qr . W_qb^T)[h*128 .. h*128 + 128)                  per index head h
 *   k       = LayerNorm(x . W_k^T) = (v - mean) / sqrt(var + eps) * ln_gamma + ln_beta
 *   channels 64 + 2i, 65 + 2i of q[h] and k turn by the angle of rope_cos[p][i], rope_sin[p][i]
 *   (zeros when p is outside the tables); with rotate = 1, q[h] and k then become H v / sqrt(128),
 *   H the Sylvester Hadamard matrix (the same map on both: every q . k is unchanged)
 *   weights[h] = (x . W_proj^T)[h] / sqrt(n_heads * 128)
 *
 * The products accumulate in fp32; q_index and k_index are rounded to bf16, weights stay fp32.
 * The V4 page's INT8 quantisation of the query is not applied (sfa_indexer_scores takes bf16).
 *
 *   x           bf16 (T, H)          qr          bf16 (T, Q)
 *   w_idx_qb    bf16 (n_heads*128, Q)              w_idx_k     bf16 (128, H)
 *   ln_gamma_k, ln_beta_k  bf16 (128)             w_idx_proj  bf16 (n_heads, H)
 *   positions   int32 (T)            rope_cos, rope_sin  fp32 (rope_positions, 32)
 *   q_index     bf16 (T*n_heads, 128): sfa_indexer_scores' q_index
 *   k_index     bf16 (T, 128): the new rows of its index-key cache
 *   weights     fp32 (T, n_heads): sfa_indexer_scores' weights
 *   workspace   >= sfa_indexer_prolog_workspace_size bytes, 256-byte aligned, no initialisation
 *
 * Errors as sfa_mla_prolog's. With T = 0 nothing is read or queued and the pointers may be NULL.
 */
typedef struct {
  int32_t tokens;               /* T >= 0                                                     */
  int32_t hidden;               /* H: a multiple of 64 in [256, 65536]                        */
  int32_t q_lora_rank;          /* Q: a multiple of 64 in [256, 4096]                         */
  int32_t n_heads;              /* index heads: must be 64                                    */
  int32_t head_dim;             /* must be 128                                                */
  int32_t rope_positions;       /* rows of rope_cos and rope_sin, >= 1                        */
  int32_t rotate;               /* 0, or 1: the Hadamard transform of query and key           */
  float eps;                    /* LayerNorm epsilon, finite and >= 0                         */
} sfa_indexer_prolog_dims;

int sfa_indexer_prolog_workspace_size(const sfa_indexer_prolog_dims* dims, size_t* bytes_out);
int sfa_indexer_prolog(const sfa_indexer_prolog_dims* dims, const void* x, const void* qr, const void* w_idx_qb,
                       const void* w_idx_k, const void* ln_gamma_k, const void* ln_beta_k, const void* w_idx_proj,
                       const int32_t* positions, const float* rope_cos, const float* rope_sin, void* q_index,
                       void* k_index, float* weights, void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SFA_H_ */
