/*
 * mla.h -- C ABI of the token-sparse MLA decode library (libmla.so, gfx950 / MI355X).
 *
 * What the library computes: Multi-head Latent Attention decode in absorbed form, where every query
 * head of a row attends over one shared 512-dim latent per selected token and the value is that same
 * latent (page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic intensity"; page
 * "flops/attn-mla-kernel-support-matrix", section "Workarounds"). Tokens live in a quantized, paged
 * cache of per-token records and are picked by an indices tensor of shape (batch, seq_len_q, topk)
 * whose negative entries are ignored (page "flops/flashmla-decode-fp8-fp4-kv", section "Workarounds";
 * page "deepseek-ai/FlashMLA", section "Key technical details").
 *
 * Call sequence (page "deepseek-ai/FlashMLA", section "How to use it"): obtain the tile-scheduler
 * metadata once with mla_get_metadata, then call mla_sparse_decode for every generation step.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers; "host" pointers are ordinary host memory.
 *   - Tensors are dense and row-major in the shapes given; R = batch * seq_len_q query rows.
 *   - The caller allocates and owns every buffer. The library allocates nothing, keeps no state
 *     between calls and may be called from several host threads.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL = default
 *     stream). Device-side results are valid once the stream reaches that point.
 *   - Errors are returned as negative mla_status codes; nothing throws across the ABI. Argument
 *     checks happen on the host before anything is enqueued, so a failed call enqueues nothing.
 *     A fault inside a kernel (for example an out-of-pool index) surfaces at the caller's next
 *     synchronisation of the stream.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_HEAD_DIM 512          /* latent dim = d_qk = d_v */
#define MLA_FP8_RECORD_BYTES 528  /* 512 e4m3 values, then 16 e8m0 scales (one per 32 values) */
#define MLA_FP4_RECORD_BYTES 288  /* 256 bytes of e2m1 (even index in the low nibble), then 32 e4m3
                                     scales (one per 16 values) */
#define MLA_TILE_TOKENS 64        /* token slots per scheduling unit */
#define MLA_SCHED_FIELDS 8        /* int32 fields per part in the schedule */
#define MLA_NOALLOC_SCRATCH_BYTES (72u << 20)  /* fixed split scratch of mla_sparse_decode_noalloc */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,   /* null pointer, bad shape, misaligned buffer, inconsistent arguments */
  MLA_ERR_UNSUPPORTED = -2,   /* shape outside what the kernels implement (e.g. head_dim != 512) */
  MLA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than mla_workspace_bytes() */
  MLA_ERR_INDEX_RANGE = -4,   /* mla_check_indices found an index at or past the cache size */
  MLA_ERR_HIP = -5,           /* a HIP runtime call or kernel launch failed */
  MLA_ERR_SCRATCH_LIMIT = -6  /* mla_sparse_decode_noalloc: the split partials would need more than
                                 MLA_NOALLOC_SCRATCH_BYTES */
} mla_status;

/* Human-readable text for a status code (static storage, never NULL). */
const char* mla_error_string(int code);

/*
 * Number of parts the schedule will use, computed on the host (no device work).
 * The metadata partitions the units of all rows over parts: a row owns ceil(topk/64) fp8 units then
 * ceil(extra_topk/64) fp4 units (at least one unit in all); U = R * units_per_row; the part count is
 * P_eff = max(1, min(num_parts, U / min_tiles_per_part)). num_parts == 0 selects the library's
 * default for the current device and h_q (one part per CU, divided by the number of head groups)
 * and raises min_tiles_per_part to at least 4.
 * Returns MLA_OK and writes *num_parts_used (host).
 * The pages call for "tile-scheduler metadata computed once before the decode loop" and "split
 * decoding with num_splits" (page "flops/flashmla-decode-fp8-fp4-kv", section "Workarounds"); the
 * partition rule itself is this library's own specification.
 */
int mla_metadata_parts(int batch, int seq_len_q, int h_q, int topk, int extra_topk, int num_parts,
                       int min_tiles_per_part, int* num_parts_used);

/*
 * Compute the tile-scheduler metadata on the device (one small kernel on `stream`).
 *   sched      device int32 [num_parts_used][8]: part p covers the contiguous units
 *              [floor(p*U/P_eff), floor((p+1)*U/P_eff)) and stores
 *              {begin_row, begin_tile, end_row, end_tile (exclusive end unit), first_slot, 0, 0, 0}
 *              where first_slot is the workspace slot of its split of begin_row.
 *   split_ptr  device int32 [R+1]: exclusive prefix sum of num_splits[r], the number of parts
 *              meeting row r; row r's splits use workspace slots split_ptr[r] .. split_ptr[r+1]-1.
 *   sched_capacity  number of [8]-int32 entries `sched` can hold (must be >= P_eff).
 *   num_parts_used  host out: P_eff.
 * The result depends only on the integer arguments, never on index values, so it is computed once
 * per decode loop and reused for every step.
 */
int mla_get_metadata(int batch, int seq_len_q, int h_q, int topk, int extra_topk, int num_parts,
                     int min_tiles_per_part, int32_t* sched, int sched_capacity, int32_t* split_ptr,
                     int* num_parts_used, void* stream);

/*
 * Bytes of workspace mla_sparse_decode needs for this schedule: 0 when every part starts on a row
 * boundary (no row is split, the workspace may be NULL); otherwise room for partial outputs
 * [R + P_eff - 1][h_q][512] (bf16 for h_q <= 64, fp32 above) followed by fp32 partial lse
 * [R + P_eff - 1][h_q], each 256-byte
 * aligned. Host-only; returns 0 for invalid arguments as well.
 */
size_t mla_workspace_bytes(int batch, int seq_len_q, int h_q, int topk, int extra_topk,
                           int num_parts_used);

/*
 * Sparse MLA decode: out, lse = attention of every query head over the selected tokens.
 *   q              device bf16 [batch][seq_len_q][h_q][512]; 16-byte aligned.
 *   k_cache        device uint8 [k_tokens][528] fp8 records (a paged pool viewed as flat tokens:
 *                  token id = physical_block * block_size + offset); 16-byte aligned.
 *   indices        device int32 [batch][seq_len_q][topk]: flat token ids into k_cache; entries < 0
 *                  are ignored; entries >= k_tokens are a precondition violation (not checked on
 *                  this path; see mla_validate_indices).
 *   extra_k_cache  NULL, or device uint8 [extra_tokens][288] fp4 records, used next to the fp8
 *                  k_cache (page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic
 *                  intensity"); 16-byte aligned.
 *   extra_indices  NULL, or device int32 [batch][seq_len_q][extra_topk] into extra_k_cache.
 *                  Each row attends with ONE softmax over the union of both selections.
 *   softmax_scale  multiplier of q.k before the softmax (e.g. 1/sqrt(512)); must be finite and
 *                  > 0 (MLA_ERR_INVALID_ARG otherwise). The scaled scores are computed in fp32, so
 *                  |softmax_scale * q.k| must stay within fp32 range, like the cache values'.
 *   sched, split_ptr, num_parts_used  the metadata from mla_get_metadata for the same
 *                  (batch, seq_len_q, h_q, topk, extra_topk).
 *   workspace      device buffer, 256-byte aligned, of workspace_bytes >= mla_workspace_bytes(...)
 *                  (NULL allowed when that is 0).
 *   out            device bf16 [batch][seq_len_q][h_q][512]; 8-byte aligned.
 *   lse            device fp32 [batch][seq_len_q][h_q]: natural-log log-sum-exp of the scaled scores
 *                  (page "deepseek-ai/FlashMLA", section "How to use it", output and lse).
 * A row with no valid entry gets out = 0 and lse = -inf. Rows split over several parts are merged
 * by log-sum-exp in a second kernel on the same stream.
 */
int mla_sparse_decode(const void* q, const uint8_t* k_cache, int64_t k_tokens,
                      const int32_t* indices, int topk, const uint8_t* extra_k_cache,
                      int64_t extra_tokens, const int32_t* extra_indices, int extra_topk, int batch,
                      int seq_len_q, int h_q, float softmax_scale, const int32_t* sched,
                      const int32_t* split_ptr, int num_parts_used, void* workspace,
                      size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Fused decode: Q-norm, RoPE, the sparse attention, conjugate RoPE on the output and the cast to
 * FP8, in one launch (page "deepseek-ai/FlashMLA", section "What it is": the fused kernel; section
 * "How to use it": the decode call returns FP8 outputs for a downstream FP8 einsum). Supported for
 * h_q > 64 (the 128-head kernel); MLA_ERR_UNSUPPORTED otherwise. The pages leave the details open;
 * this library's reading:
 *   q              device bf16 [batch][seq_len_q][h_q][512], the query BEFORE normalisation.
 *   q_norm_weight  device bf16 [512], 16-byte aligned: each head row becomes
 *                  q / sqrt(mean(q^2) + q_norm_eps) * q_norm_weight (RMSNorm over the 512 dims).
 *   rope_cos, rope_sin  device fp32 [batch][seq_len_q][32], 16-byte aligned: the rotary part is the
 *                  last 64 latent dims as 32 interleaved pairs (448 + 2i, 449 + 2i); pair i of row r
 *                  is rotated by the angle with cosine rope_cos[r][i] and sine rope_sin[r][i]:
 *                  (x0, x1) -> (x0 c - x1 s, x0 s + x1 c). The rotated query enters QK^T as bf16.
 *   out_fp8        device uint8 [batch][seq_len_q][h_q][528], 16-byte aligned: each output row,
 *                  with its rotary pairs rotated back ((y0, y1) -> (y0 c + y1 s, y1 c - y0 s)),
 *                  stored as an fp8 record in the cache's own format (512 e4m3 values, then 16 e8m0
 *                  scales, one per 32 values; scale 2^ceil(log2(amax / 448)), values rounded to
 *                  nearest, ties to even). A row with no valid entry stores zeros with scale bytes 127.
 *   lse            as in mla_sparse_decode (of the scores of the normalised, rotated query).
 * All other arguments, the metadata and the workspace are those of mla_sparse_decode.
 */
int mla_sparse_decode_fused(const void* q, const void* q_norm_weight, float q_norm_eps,
                            const float* rope_cos, const float* rope_sin, const uint8_t* k_cache,
                            int64_t k_tokens, const int32_t* indices, int topk,
                            const uint8_t* extra_k_cache, int64_t extra_tokens,
                            const int32_t* extra_indices, int extra_topk, int batch, int seq_len_q,
                            int h_q, float softmax_scale, const int32_t* sched,
                            const int32_t* split_ptr, int num_parts_used, void* workspace,
                            size_t workspace_bytes, uint8_t* out_fp8, float* lse, void* stream);

/*
 * Sparse MLA prefill: the same attention for s_q query tokens of one sequence, each with its own
 * selection (page "deepseek-ai/FlashMLA", section "How to use it", sparse prefill with a query
 * tensor, the KV cache and an indices tensor telling each query token which KV tokens it attends
 * to; section "What it is": the sparse kernels of both phases read the FP8/FP4 cache).
 *   q        device bf16 [s_q][h_q][512]; out device bf16 [s_q][h_q][512]; lse device fp32 [s_q][h_q].
 *   indices  device int32 [s_q][topk] flat token ids into k_cache (negative = ignored);
 *            extra_k_cache / extra_indices [s_q][extra_topk] as in mla_sparse_decode.
 * No metadata and no workspace: with many query rows, whole rows are spread evenly over the device
 * (one part per CU and head group) and no row is split. Same checks, kernels and results per row as
 * mla_sparse_decode with batch = 1, seq_len_q = s_q.
 */
int mla_sparse_prefill(const void* q, int s_q, int h_q, const uint8_t* k_cache, int64_t k_tokens,
                       const int32_t* indices, int topk, const uint8_t* extra_k_cache,
                       int64_t extra_tokens, const int32_t* extra_indices, int extra_topk,
                       float softmax_scale, void* out, float* lse, void* stream);

/*
 * mla_sparse_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. Same arguments, checks, kernels and results
 * as mla_sparse_decode, without the workspace: the split partials go to a fixed device array of
 * MLA_NOALLOC_SCRATCH_BYTES (72 MiB) that the library holds on each device it runs on until the
 * process ends. The call allocates nothing. A schedule whose partials need more than that
 * (mla_workspace_bytes(...) > MLA_NOALLOC_SCRATCH_BYTES) is refused with MLA_ERR_SCRATCH_LIMIT
 * before any device work. Calls on one device share the array: calls that overlap in time on one
 * device (different streams, or several host threads) race and must be serialised by the caller.
 */
int mla_sparse_decode_noalloc(const void* q, const uint8_t* k_cache, int64_t k_tokens,
                              const int32_t* indices, int topk, const uint8_t* extra_k_cache,
                              int64_t extra_tokens, const int32_t* extra_indices, int extra_topk,
                              int batch, int seq_len_q, int h_q, float softmax_scale,
                              const int32_t* sched, const int32_t* split_ptr, int num_parts_used,
                              void* out, float* lse, void* stream);

/*
 * Log-sum-exp merge of split partials (the second half of split decoding, page
 * "flops/flashmla-decode-fp8-fp4-kv", section "Workarounds"):
 *   partial      device fp32 [S][h_q][512]: each split's output, already normalised by its own sum.
 *   partial_lse  device fp32 [S][h_q]: each split's natural-log lse (-inf for an empty split).
 *   split_ptr    device int32 [rows+1]: row r merges slots split_ptr[r] .. split_ptr[r+1]-1.
 *   out          device bf16 [rows][h_q][512]; lse device fp32 [rows][h_q].
 * For each (row, head): M = max lse_i, w_i = exp(lse_i - M), lse = M + log(sum w_i),
 * out = sum w_i o_i / sum w_i; a row whose splits are all empty gets out = 0, lse = -inf.
 */
int mla_combine(const float* partial, const float* partial_lse, const int32_t* split_ptr, int rows,
                int h_q, void* out, float* lse, void* stream);

/*
 * Cache writer: quantize bf16 latents into the cache's per-token records (the step before decode).
 *   x             device bf16 [n][512], 16-byte aligned: one latent per new token.
 *   slots         NULL (row i is written to token i, n <= cache_tokens), or device int32 [n]: the
 *                 flat token id (physical_block * block_size + offset) each row is written to;
 *                 entries < 0 or >= cache_tokens write nothing.
 *   record_bytes  528 (fp8 records) or 288 (fp4 records); cache device uint8 [cache_tokens][record],
 *                 16-byte aligned.
 * Layouts (page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic intensity"; page
 * "deepseek-ai/FlashMLA", section "Key technical details": quantized values first, then the
 * token's scales): fp8 = 512 e4m3 values then 16 e8m0 scales, one per 32 values; fp4 = 256 bytes of
 * e2m1 (even index in the low nibble) then 32 e4m3 scales, one per 16 values. The pages leave the
 * choice of scales open; this library's rule: fp8 block with a = max|x|: scale 2^k with
 * k = ceil(log2(a / 448)) clipped to [-127, 127] (k = 0 for an all-zero block), values rounded to the
 * nearest e4m3 of x / 2^k, ties to even; fp4 block: scale = the nearest e4m3 of a / 6 (ties to even,
 * saturating at 448; 1.0 when it rounds to 0), values the nearest e2m1 of x / scale (ties to even,
 * saturating at +-6). Rounding keeps the sign. x must be finite. Distinct rows must not share a slot
 * (the record written last is unspecified).
 */
int mla_quantize_records(const void* x, int64_t n, const int32_t* slots, int record_bytes,
                         uint8_t* cache, int64_t cache_tokens, void* stream);

/*
 * Diagnostic: dequantize whole records with the same device routine the decode kernel uses.
 *   cache         device uint8 records of record_bytes (528 = fp8, 288 = fp4); 16-byte aligned.
 *   idx           device int32 [n] token ids (all must be >= 0 and inside the cache).
 *   out_bf16      device bf16 [n][512].
 */
int mla_dequant_records(const uint8_t* cache, int record_bytes, const int32_t* idx, int n,
                        void* out_bf16, void* stream);

/*
 * Debug helper: count the entries of idx[0..n) that are >= num_tokens (negative entries are
 * "ignored" entries and are not counted). Writes the count to *bad_count (device int32).
 */
int mla_validate_indices(const int32_t* idx, int64_t n, int64_t num_tokens, int32_t* bad_count,
                         void* stream);

/*
 * Debug helper, blocking form of mla_validate_indices: runs the same count into bad_count (device
 * int32), waits for `stream`, and returns MLA_OK when every entry is < num_tokens (negative entries
 * are ignored entries and always pass) or MLA_ERR_INDEX_RANGE when some entry is out of the cache.
 * Out-of-cache indices are a precondition violation of mla_sparse_decode (page "deepseek-ai/FlashMLA",
 * section "Key technical details": entries select KV pages, -1 marks the ignored ones); this call
 * lets a caller test that precondition off the hot path.
 */
int mla_check_indices(const int32_t* idx, int64_t n, int64_t num_tokens, int32_t* bad_count,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
