/*
 * mla.h - C ABI of the MI355X (gfx950) paged / sparse MLA decode library (libmla.so).
 *
 * Multi-head latent attention decode: every query head attends over one
 * shared 576-wide latent row per cached token (512 latent dims + 64 RoPE
 * dims); the row's first 512 dims are the value ("[flashinfer] FlashInfer,
 * NVFP4를 활용한 DeepSeek-V4 디코딩 성능 최적화", section "코드 분석", item 2:
 * paged MQA over a latent row that is both K and V).  Scores are
 * softmax_scale * q.k over all 576 dims; O = softmax(scores) V; the returned
 * LSE is the natural log of the softmax denominator, fp32 (same README
 * table).  Queries that see no token get O = 0 and LSE = -inf.
 *
 * Conventions for every call below:
 *  - Pointers marked [device] are device pointers, [host] host pointers.
 *    Tensors are dense and row-major.  q, kcache, kv, out and workspace must
 *    be 16-byte aligned.
 *  - The caller allocates and owns every buffer and the stream.  The library
 *    allocates nothing, keeps no state between calls and never synchronises
 *    (mla_decode_paged_noalloc aside, whose workspace is an array the library
 *    holds on each GPU).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    All work is enqueued on it asynchronously.
 *  - Arguments the host can check are validated before anything is
 *    launched; a bad argument returns an error status and enqueues nothing.
 *    Values that live in device memory (block-table entries, sequence
 *    lengths, indices) are the caller's responsibility: an out-of-range
 *    value there is undefined behaviour.  Device faults surface at the
 *    caller's next synchronisation.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_D_QK 576           /* dims of a cached latent row: 512 latent + 64 RoPE */
#define MLA_D_V 512            /* value dims: the first 512 dims of the same row    */
#define MLA_PAGE 64            /* tokens per KV-cache page                          */
#define MLA_SPARSE_REC 640     /* bytes per fp8 record of the sparse cache          */
#define MLA_META_INTS 8        /* int32 per part in the tile-scheduler metadata     */
#define MLA_MAX_BATCH_META 16384 /* largest batch mla_get_metadata accepts          */

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, misalignment, non-finite scale */
    MLA_ERR_UNSUPPORTED = 2,   /* a shape outside what the kernels handle             */
    MLA_ERR_WORKSPACE = 3,     /* workspace_bytes smaller than the size function's value */
    MLA_ERR_HIP = 4            /* the HIP runtime refused a launch                     */
} mla_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(mla_status_t status);

/*
 * Number of KV parts the tile scheduler splits one decode step into: about
 * one workgroup per compute unit once the row groups of a sequence are
 * counted (64-row groups up to 64 rows, 128-row groups beyond), two per
 * compute unit when 32 < s_q*h_q <= 64.  num_cus <= 0 queries the current
 * device.  Returns >= 1; up to 64 rows a multiple of 8 when num_cus is (each
 * XCD then holds whole parts), above 64 rows num_cus / (128-row groups)
 * (the parts beyond the last multiple of 8 fill the compute units left over).
 * Any value >= 1 is valid for the calls below; larger values force more KV
 * splits.
 */
int mla_num_parts(int num_cus, int h_q, int s_q);

/*
 * Tile-scheduler metadata, computed on the device from the device-resident
 * sequence lengths, once per decode step and reused by every layer
 * ("Qu'est-ce que FlashMLA ?", section "Installation et utilisation de
 * FlashMLA", steps 2-3: get_mla_metadata, then one decode call per layer).
 *
 *   cache_seqlens [device] int32[batch]  tokens in each sequence's cache,
 *                                        including its s_q new query tokens
 *   tile_meta     [device] int32[num_parts * MLA_META_INTS]  (out)
 *   num_splits    [device] int32[batch + 1]                  (out)
 *
 * Work is counted in 64-token blocks, plus a fixed cost per non-empty
 * sequence (none for s_q*h_q <= 64 rows, four blocks above), and cut into
 * num_parts contiguous, equally sized ranges of the flattened (sequence,
 * block) order; a sequence crossing a range edge is split.
 * num_splits is the exclusive prefix sum of the number of parts touching
 * each sequence (num_splits[b+1] - num_splits[b] = splits of sequence b);
 * it indexes the partial results in the workspace.  tile_meta[p] holds
 * {begin_seq, begin_block, end_seq, end_block, first_partial_slot, 0,0,0}.
 * h_q and s_q (the call shape of the pages' API) choose that fixed cost;
 * the decode result does not depend on the partition.
 * batch <= MLA_MAX_BATCH_META.
 */
mla_status_t mla_get_metadata(const int32_t* cache_seqlens, int batch, int h_q, int s_q,
                              int num_parts, int32_t* tile_meta, int32_t* num_splits,
                              void* stream);

/* The same partition computed on the host from host arrays ([host] pointers, synchronous). */
mla_status_t mla_get_metadata_host(const int32_t* cache_seqlens, int batch, int h_q, int s_q,
                                   int num_parts, int32_t* tile_meta, int32_t* num_splits);

/* Bytes of workspace mla_decode_paged needs (split-KV partial outputs and LSEs). */
size_t mla_workspace_size(int batch, int s_q, int h_q, int num_parts);

/*
 * Paged MLA decode ("Qu'est-ce que FlashMLA ?", step 3: flash_mla_with_kvcache
 * with q, kvcache, block_table, cache_seqlens, dv, metadata, num_splits,
 * causal; "DeepSeek, FlashMLA 오픈소스 공개", summary: BF16, 64-token pages).
 *
 *   q             [device] bf16 [batch, s_q, h_q, 576]
 *   kcache        [device] bf16 [num_blocks, 64, 1, 576]
 *   block_table   [device] int32[batch, max_blocks]; logical token t of
 *                 sequence b is row t % 64 of page block_table[b][t / 64]
 *   cache_seqlens [device] int32[batch]; must equal what the metadata saw
 *   softmax_scale fp32 multiplier of q.k (e.g. 576^-0.5)
 *   causal        nonzero: the s_q queries are the sequence's last s_q
 *                 tokens and query s sees tokens <= L - s_q + s ("[flashinfer]
 *                 ...", README: causal mask against the request's last tokens)
 *   tile_meta, num_splits, num_parts: from mla_get_metadata
 *   workspace     [device] >= mla_workspace_size(batch, s_q, h_q, num_parts) bytes
 *   out           [device] bf16 [batch, s_q, h_q, 512]   (written)
 *   lse           [device] fp32 [batch, s_q, h_q], natural log (written)
 *
 * Rows past a sequence's end and block-table slots past its last page are
 * never used, whatever they hold.  s_q * h_q <= 4096.
 */
mla_status_t mla_decode_paged(const void* q, const void* kcache, int64_t num_blocks,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                              float softmax_scale, int causal,
                              const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                              void* workspace, size_t workspace_bytes,
                              void* out, float* lse, void* stream);

/*
 * mla_decode_paged without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It takes the same arguments as mla_decode_paged except
 * workspace and workspace_bytes, and computes the same result with the same
 * kernels.  The split-KV partials go to an array of MLA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on (from the library's load to
 * the end of the process); the call allocates and frees nothing.
 *
 *  - The array used is the current device's (hipGetDevice); `stream` must
 *    belong to that device.  Its address is looked up on the first call on a
 *    device.
 *  - A shape whose workspace (mla_workspace_size(batch, s_q, h_q, num_parts))
 *    exceeds MLA_NOALLOC_SCRATCH_BYTES returns MLA_ERR_WORKSPACE before
 *    anything is launched; 32 MiB holds the partials of s_q * h_q = 16 rows for
 *    batch + num_parts up to 1022.  Other argument errors are those of
 *    mla_decode_paged.
 *  - Nothing in the array needs to start at zero.  Every call on one GPU shares
 *    its array, which keeps the last call's partials: calls that overlap in
 *    time on one GPU (two streams, two threads) race and give undefined
 *    results.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
mla_status_t mla_decode_paged_noalloc(const void* q, const void* kcache, int64_t num_blocks,
                                      const int32_t* block_table, int max_blocks,
                                      const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                      float softmax_scale, int causal,
                                      const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                      void* out, float* lse, void* stream);

/*
 * Paged decode in the DeepSeek-V4 main-attention geometry ("[flashinfer]
 * FlashInfer, NVFP4를 활용한 DeepSeek-V4 디코딩 성능 최적화", README: paged MQA over
 * one 512-wide latent row per token that is both K and V, 64-token pages,
 * q_len query tokens per request with the causal mask against the request's
 * last tokens, an optional per-head attention sink, bf16 output, natural-log
 * fp32 LSE), here over a bf16 cache.
 *
 *   q        [device] bf16 [batch, s_q, h_q, 512]
 *   kcache   [device] bf16 [num_blocks, 64, 512]; the row is K, and V
 *   sinks    [device] fp32 [h_q] or NULL: one more logit per head in the
 *            softmax denominator, carrying no value, in the units of the
 *            scaled scores (not multiplied by softmax_scale); the returned
 *            LSE is the log of the whole denominator (a row that sees no
 *            token gets O = 0, LSE = its sink)
 *
 * Metadata, block table, lengths, causal rule, workspace size
 * (mla_workspace_size) and outputs are as for mla_decode_paged; any finite
 * softmax_scale (e.g. 512^-0.5).
 */
mla_status_t mla_decode_paged_latent512(const void* q, const void* kcache, int64_t num_blocks,
                                       const int32_t* block_table, int max_blocks,
                                       const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                       float softmax_scale, int causal, const float* sinks,
                                       const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                       void* workspace, size_t workspace_bytes,
                                       void* out, float* lse, void* stream);

/*
 * The DeepSeek-V4 decode geometry over an FP4 cache ("[flashinfer] FlashInfer,
 * NVFP4를 활용한 DeepSeek-V4 디코딩 성능 최적화", README tensor table: kv_cache
 * [num_pages, 64, 256] packed E2M1, kv_scale [num_pages, 64, 32] UE4M3 block-16
 * scales; "deepseek-ai/FlashMLA" project summary, section 기술적 세부 사항:
 * e2m1 caches).  The query stays bf16.
 *
 *   kv_codes  [device] uint8[num_blocks, 64, 256]: the 512 values of a token's
 *             latent row as OCP E2M1 nibbles, value 2j in the low nibble of
 *             byte j and value 2j+1 in the high nibble
 *   kv_scales [device] uint8[num_blocks, 64, 32]: byte b is the scale of
 *             values 16b..16b+15, decoded as an E4M3FN byte (valid UE4M3
 *             scales have the top bit clear).  Value = e2m1 * scale, exactly.
 *
 * q, sinks, metadata, block table, lengths, causal rule, workspace size
 * (mla_workspace_size) and outputs are as for mla_decode_paged_latent512.
 * Both cache pointers must be 16-byte aligned.  Rows are addressed with
 * 64-bit offsets: the cache may fill the device.
 */
mla_status_t mla_decode_paged_fp4(const void* q, const void* kv_codes, const void* kv_scales, int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  float softmax_scale, int causal, const float* sinks,
                                  const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                  void* workspace, size_t workspace_bytes,
                                  void* out, float* lse, void* stream);

/*
 * The fused decode ("deepseek-ai/FlashMLA" project summary, section 개요 bullet 3: one
 * kernel launch merges the query norm, RoPE, the attention, the conjugate RoPE on the output
 * side and the final cast to FP8; section 사용 방법 step 5: its FP8 output feeds the FP8 einsum
 * that follows), here on the DeepSeek-V4 decode geometry of mla_decode_paged_latent512 /
 * mla_decode_paged_fp4.  Per query row (token s of sequence b, head h):
 *
 *   q'  = RoPE(q * norm_weight / sqrt(mean(q^2) + norm_eps))      (RMS norm over 512 dims)
 *   O   = the paged decode of q' (causal rule, sinks: mla_decode_paged_latent512)
 *   O'  = conjugate RoPE(O)
 *   out = e4m3 codes of O' / scale, scale = max(max|O'|, 2^-126) / 448 (one fp32 per row)
 *
 * RoPE turns the interleaved pairs of dims (448 + 2i, 449 + 2i), i < 32, by the query token's
 * angle theta_i; the conjugate RoPE turns the same pairs of O by -theta_i.  (The cached rows'
 * last 64 dims carry their own tokens' rotations, written when the cache was filled.)  The
 * codes are OCP E4M3FN, rounded to nearest even from fp32 x * (1 / scale).
 *
 *   q           [device] bf16 [batch, s_q, h_q, 512]: the query before its norm and RoPE
 *   kv_codes    [device] bf16 [num_blocks, 64, 512] when kv_scales is NULL; otherwise
 *               uint8 [num_blocks, 64, 256] FP4 codes (as mla_decode_paged_fp4)
 *   kv_scales   [device] uint8 [num_blocks, 64, 32] UE4M3 block scales, or NULL (bf16 pages)
 *   norm_weight [device] fp32 [512], shared by the heads; norm_eps >= 0
 *   rope_cs     [device] fp32 [batch, s_q, 64]: cos(theta_i), i < 32, then sin(theta_i), of
 *               each query token
 *   out_fp8     [device] uint8 [batch, s_q, h_q, 512] e4m3 codes (written)
 *   out_scale   [device] fp32 [batch, s_q, h_q] (written); lse as for mla_decode_paged
 *
 * Block table, lengths, causal rule, sinks, metadata and workspace (mla_workspace_size) are as
 * for mla_decode_paged_latent512.  norm_weight and rope_cs must be 16-byte aligned.
 */
mla_status_t mla_decode_fused(const void* q, const void* kv_codes, const void* kv_scales, int64_t num_blocks,
                              const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                              int batch, int s_q, int h_q, float softmax_scale, int causal, const float* sinks,
                              const float* norm_weight, float norm_eps, const float* rope_cs,
                              const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                              void* workspace, size_t workspace_bytes,
                              void* out_fp8, float* out_scale, float* lse, void* stream);

/*
 * Paged MLA decode over an fp8 cache: the same call as mla_decode_paged with
 * the cache in the fp8 layout of the decode path ("deepseek-ai/FlashMLA"
 * project summary, section 사용 방법 step 3: flash_mla_with_kvcache on the
 * FP8 KV cache; section 기술적 세부 사항: raw e4m3 values plus a per-token
 * scale).
 *
 *   kcache   [device] uint8[num_blocks, 64, 640]: 64-token pages of records,
 *            bytes [0,576) the OCP E4M3FN codes of the row's 576 dims,
 *            bytes [576,580) the token's fp32 scale (little endian),
 *            bytes [580,640) unused.  Row value = e4m3(code) * scale.
 *
 * Every other argument, the workspace size and the result are as for
 * mla_decode_paged.  Records are addressed with 64-bit offsets: the cache
 * may fill the device.
 */
mla_status_t mla_decode_paged_fp8(const void* q, const void* kcache, int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  float softmax_scale, int causal,
                                  const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                  void* workspace, size_t workspace_bytes,
                                  void* out, float* lse, void* stream);

/*
 * Number of topk splits mla_decode_sparse uses per query token for a given
 * shape when called with splits = 0, and the workspace it then needs.  The
 * rule: as many splits as keep the work items (query tokens x row groups x
 * splits) within one round of 256, at least one, at most topk / 32, and at
 * least topk / 2048.
 */
int mla_sparse_splits(int batch, int s_q, int h_q, int topk);
size_t mla_workspace_size_sparse(int batch, int s_q, int h_q, int topk, int splits);

/*
 * Sparse fp8 MLA decode ("deepseek-ai/FlashMLA" project summary, sections
 * "사용 방법" and "기술적 세부 사항": token-level sparse attention over an fp8
 * cache holding raw quantised values plus a per-token scale; a 3-D indices
 * tensor lists the tokens each query reads, -1 entries are ignored).
 *
 *   q        [device] bf16 [batch, s_q, h_q, 576]
 *   kv       [device] uint8[num_tokens, 640] records: bytes [0,576) are OCP
 *            E4M3FN codes of the 576 dims, bytes [576,580) the token's fp32
 *            scale (little endian), bytes [580,640) unused.  Row value =
 *            e4m3(code) * scale.
 *   indices  [device] int32[batch, s_q, topk]: global token rows in
 *            [0, num_tokens), or -1 to skip.  Records are addressed with
 *            64-bit offsets: the pool may fill the device.  Each entry is one term
 *            (a repeated row counts repeatedly).  There is no causal flag:
 *            the index lists carry any masking.
 *   splits   0 = mla_sparse_splits(...); otherwise topk is cut into this many
 *            ranges (clamped to [1, ceil(topk/32)]) merged by an LSE combine
 *   workspace[device] >= mla_workspace_size_sparse(batch, s_q, h_q, topk, splits)
 *   out, lse as for mla_decode_paged.
 */
mla_status_t mla_decode_sparse(const void* q, const void* kv, int64_t num_tokens,
                               const int32_t* indices, int topk,
                               int batch, int s_q, int h_q, float softmax_scale, int splits,
                               void* workspace, size_t workspace_bytes,
                               void* out, float* lse, void* stream);

/*
 * Sparse prefill ("deepseek-ai/FlashMLA" project summary, section "사용 방법"
 * step 2: flash_mla_sparse_fwd(q, kv, indices, ...) takes the query tensor,
 * the KV cache and a 3-D indices tensor naming the KV tokens each query token
 * reads; section "기술적 세부 사항": quantised caches, -1 entries ignored).
 * Every query token of a prompt chunk attends its own index list over the
 * same fp8 record pool as mla_decode_sparse; one latent head (h_kv = 1).
 *
 *   q        [device] bf16 [s_q, h_q, 576]  (s_q query tokens)
 *   kv       [device] uint8[num_tokens, 640] records, as for mla_decode_sparse
 *   indices  [device] int32[s_q, topk] (the [s_q, 1, topk] tensor of one
 *            latent head), rows in [0, num_tokens) or -1 to skip
 *   splits, workspace (mla_workspace_size_sparse(1, s_q, h_q, topk, splits))
 *            as for mla_decode_sparse
 *   out      [device] bf16 [s_q, h_q, 512]; lse [device] fp32 [s_q, h_q]
 *
 * The result is that of mla_decode_sparse with batch = 1 (same kernels: one
 * work item per query token and 64 heads).  s_q <= 2^24, h_q <= 4096.
 */
mla_status_t mla_sparse_prefill(const void* q, const void* kv, int64_t num_tokens,
                                const int32_t* indices, int topk, int s_q, int h_q,
                                float softmax_scale, int splits,
                                void* workspace, size_t workspace_bytes,
                                void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
