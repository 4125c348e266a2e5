// Internal declarations shared by the host API (mla_api.cpp) and the gfx950 kernels (mla_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include "mla.h"
#include <cstdint>

namespace mla {

constexpr int kDqk = 576;            // latent (512) + RoPE (64) dims of one cached row
constexpr int kDv = 512;             // value dims (first 512 of the row)
constexpr int kPage = 64;            // tokens per page
constexpr int kRec = 640;            // bytes per sparse fp8 record
constexpr int kChunk = 32;           // tokens per kernel chunk
constexpr int kMetaInts = 8;
constexpr int kMaxBatchMeta = 16384;
constexpr int kMaxRows = 4096;       // s_q * h_q limit
constexpr int kSparseTargetItems = 256;   // work items (one per compute unit) sparse splitting aims for
constexpr int kMaxSparseSplit = 2048;     // index entries one sparse split may hold

// Wave pairs (32 query rows each) per workgroup of the large-row decode kernel, used for
// s_q*h_q (paged) or h_q (sparse) above 16 rows: one pair (and two token streams) up to 32
// rows, two pairs (64 rows per workgroup) beyond.
inline __host__ __device__ int big_pairs(int rows) { return rows <= 32 ? 1 : 2; }

// Row tiling of one sequence's s_q*h_q query rows.  A workgroup holds 4 waves:
// `rw` of them split the rows (16*nt rows each), the other factor 4/rw splits
// the KV chunks between independent softmax streams merged at the end.
struct Tiling {
    int nt;          // 16-row MFMA tiles per wave (1 or 2)
    int rw;          // row-waves per workgroup (1, 2 or 4)
    int rows_wg;     // rows per workgroup = 16 * nt * rw
    int row_groups;  // workgroups per sequence (or per sparse query token)
};
Tiling choose_tiling(int rows);

struct AttnArgs {
    const void* q;              // bf16 [groups, M, 576]
    const void* kv;             // paged: bf16 [blocks, 64, 576]; sparse: [tokens, 640] records
    const int32_t* block_table; // paged
    const int32_t* seqlens;     // paged
    const int32_t* indices;     // sparse [groups, topk]
    const int32_t* tile_meta;   // paged
    const int32_t* num_splits;  // paged: prefix [batch+1]
    void* out;                  // bf16 [groups, M, 512]
    float* lse;                 // [groups, M]
    float* part_o;              // [slots, M, 512]
    float* part_lse;            // [slots, M]
    int batch;                  // paged: sequences; sparse: query tokens (batch*s_q)
    int s_q, h_q, M;            // M = rows per group (paged s_q*h_q, sparse h_q)
    int max_blocks;
    int topk;
    int causal;
    int num_parts;              // paged parts; sparse: splits per query token
    int split_len;              // sparse entries per split (multiple of kChunk)
    int64_t kv_rows;            // sparse: records in the pool; paged fp8: pages * 64
    int kv_fp8;                 // paged: 1 = 64-token pages of 640-byte fp8 records
    int kv_fp4;                 // paged: 1 = 64-token pages of 512-wide FP4 rows (kv: 256 code
                                // bytes per token, kv_scale: 32 UE4M3 bytes per token)
    const void* kv_scale;       // FP4 pages: uint8 [blocks, 64, 32]
    int d_qk;                   // paged bf16: row width, 576 or 512 (latent row that is K and V)
    const float* sinks;         // per-head attention sinks [h_q] (natural log), or null
    float scale_log2;           // softmax_scale * log2(e)
    // fused decode (512-wide rows): the query's RMS norm and RoPE before the attention, the
    // conjugate RoPE and the FP8 cast of the output after it; out then holds e4m3 codes
    // (uint8 [groups, M, 512]) and out_scale their fp32 scale per row
    int fused;
    const float* qn_weight;     // fp32 [512]
    float qn_eps;
    const float* rope_cs;       // fp32 [batch, s_q, 64]: cos of the 32 pair angles, then sin
    float* out_scale;           // fp32 [groups, M]
};
// rotary dims of the fused decode: the interleaved pairs (448 + 2i, 449 + 2i) of the 512-wide row
constexpr int kRopeStart = 448;
constexpr float kE4m3Max = 448.f;

hipError_t launch_metadata(const int32_t* seqlens, int batch, int num_parts, int overhead,
                           int32_t* tile_meta, int32_t* num_splits, hipStream_t stream);
void metadata_host(const int32_t* seqlens, int batch, int num_parts, int overhead,
                   int32_t* tile_meta, int32_t* num_splits);
hipError_t launch_decode(const AttnArgs& a, bool sparse, hipStream_t stream);
hipError_t launch_decode_big(const AttnArgs& a, bool sparse, hipStream_t stream);
hipError_t launch_decode_rows(const AttnArgs& a, bool sparse, hipStream_t stream);
hipError_t launch_decode_m16_fp8(const AttnArgs& a, hipStream_t stream);
hipError_t launch_decode_wide(const AttnArgs& a, hipStream_t stream);
// query rows per workgroup of the one-wave-per-SIMD kernel (used above 64 rows)
constexpr int kWideRows = 128;
constexpr int kWideMinRows = 64;
// Per-sequence fixed cost in the tile scheduler's partition, in 64-token blocks: none up to 64
// rows (equal sequences then split into equal parts with one segment each), four above, where a
// segment start (Q, the first chunks, the epilogue of 128-row workgroups) costs about as much as
// that many blocks of the chunk loop.
inline int meta_overhead_blocks(long long rows) { return rows > kWideMinRows ? 4 : 0; }
// Supplies the workspace of a call that brings none: given the bytes the call needs, sets the
// pointer and size of the library's own array, or returns an error status.
typedef mla_status_t (*ScratchSource)(size_t need, void** ptr, size_t* bytes);
// mla_decode_paged with the workspace taken from `scratch` after the host-side checks pass
mla_status_t decode_paged_scratch(const void* q, const void* kcache, int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  float softmax_scale, int causal,
                                  const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                  void* out, float* lse, void* stream, ScratchSource scratch);
// whether launch_decode runs the one-wave-per-SIMD kernel, whose partials are bf16
bool decode_uses_wide(const AttnArgs& a, bool sparse);
hipError_t launch_combine(const float* part_o, const float* part_lse, const int32_t* num_splits_prefix,
                          int uniform_splits, int groups, int rows, void* out, float* lse,
                          hipStream_t stream, const float* sinks = nullptr, int h_q = 1,
                          bool bf16_parts = false);
// the combine of the fused decode: merged rows get the conjugate RoPE and the FP8 cast
hipError_t launch_combine_fused(const AttnArgs& a, hipStream_t stream);

}  // namespace mla
