// Host side of libmla.so: argument validation, workspace carving, launches, and the host
// twin of the tile-scheduler metadata.  Nothing here allocates device memory or synchronises.
#include "mla.h"
#include "mla_internal.h"

#include <cmath>
#include <cstdint>
#include <vector>

namespace {

using mla::Tiling;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int sparse_split_len(int topk, int splits) {
    const int chunks = (topk + mla::kChunk - 1) / mla::kChunk;
    const int per = (chunks + splits - 1) / splits;
    return per * mla::kChunk;
}

// number of splits actually used (no empty ranges)
int sparse_effective_splits(int topk, int splits) {
    const int len = sparse_split_len(topk, splits);
    return (topk + len - 1) / len;
}

int sparse_min_splits(int topk) { return (topk + mla::kMaxSparseSplit - 1) / mla::kMaxSparseSplit; }

int sparse_auto_splits(int batch, int s_q, int h_q, int topk) {
    const long long sets = (long long)batch * s_q;
    const Tiling t = mla::choose_tiling(h_q);
    const long long per_set = sets * t.row_groups;
    // as many splits as fit in one round of work items: a second, partly filled round costs as
    // much as it saves, and every split adds partial traffic and a combine
    long long want = mla::kSparseTargetItems / per_set;
    if (want < 1) want = 1;
    const int max_splits = (topk + mla::kChunk - 1) / mla::kChunk;
    if (want < sparse_min_splits(topk)) want = sparse_min_splits(topk);
    if (want > max_splits) want = max_splits;
    return (int)want;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// the fused decode's extra arguments
struct FusedParams {
    const float* weight;
    float eps;
    const float* rope_cs;
    float* out_scale;
};

size_t partial_bytes(long long slots, long long rows) {
    return align256((size_t)slots * rows * mla::kDv * sizeof(float)) + align256((size_t)slots * rows * sizeof(float));
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t s) {
    switch (s) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
        case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
        case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
        case MLA_ERR_HIP: return "MLA_ERR_HIP";
    }
    return "MLA_ERR_UNKNOWN";
}

int mla_num_parts(int num_cus, int h_q, int s_q) {
    if (num_cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || num_cus <= 0)
            num_cus = 256;
    }
    long long rows = (long long)(h_q > 0 ? h_q : 1) * (s_q > 0 ? s_q : 1);
    if (rows > mla::kMaxRows) rows = mla::kMaxRows;
    const Tiling t = mla::choose_tiling((int)rows);
    // One workgroup per CU.  16 < rows <= 64 (the row-split kernels): two rounds of shorter
    // parts, which even out the varying part lengths of ragged batches.  More rows (the
    // one-wave-per-SIMD kernel's 128-row groups): one round, because every extra split of a
    // sequence writes and reads back fp32 partials of all its rows (measured on the 256- and
    // 384-row workloads: one round with fewer splits is 10-20% faster than two).
    // The row-split and 16-row kernels take a multiple of 8 parts (each XCD then holds whole
    // parts); the one-wave-per-SIMD kernel places the parts beyond the last multiple of 8 on the
    // compute units left over (384 rows: 85 parts in 255 workgroups instead of 80 in 240).
    const bool wide = rows > mla::kWideMinRows;
    const int row_groups = wide ? (int)((rows + mla::kWideRows - 1) / mla::kWideRows) : t.row_groups;
    int p = (wide ? 1 : rows > 32 ? 2 : 1) * num_cus / row_groups;
    if (p >= 8 && !wide) p -= p % 8;
    return p >= 1 ? p : 1;
}

size_t mla_workspace_size(int batch, int s_q, int h_q, int num_parts) {
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_parts <= 0) return 0;
    return partial_bytes((long long)batch + num_parts, (long long)s_q * h_q);
}

int mla_sparse_splits(int batch, int s_q, int h_q, int topk) {
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || topk <= 0) return 1;
    return sparse_effective_splits(topk, sparse_auto_splits(batch, s_q, h_q, topk));
}

size_t mla_workspace_size_sparse(int batch, int s_q, int h_q, int topk, int splits) {
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || topk <= 0) return 0;
    if (splits <= 0) splits = sparse_auto_splits(batch, s_q, h_q, topk);
    const int max_splits = (topk + mla::kChunk - 1) / mla::kChunk;
    if (splits > max_splits) splits = max_splits;
    if (splits < sparse_min_splits(topk)) splits = sparse_min_splits(topk);
    const int eff = sparse_effective_splits(topk, splits);
    if (eff <= 1) return 0;
    return partial_bytes((long long)batch * s_q * eff, h_q);
}

static mla_status_t check_meta_args(const int32_t* seqlens, int batch, int num_parts,
                                    const int32_t* tile_meta, const int32_t* num_splits) {
    if (!seqlens || !tile_meta || !num_splits) return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || num_parts <= 0) return MLA_ERR_INVALID_ARG;
    if (batch > mla::kMaxBatchMeta) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

mla_status_t mla_get_metadata(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int num_parts,
                              int32_t* tile_meta, int32_t* num_splits, void* stream) {
    const mla_status_t st = check_meta_args(cache_seqlens, batch, num_parts, tile_meta, num_splits);
    if (st != MLA_OK) return st;
    const int ovh = mla::meta_overhead_blocks((long long)h_q * s_q);
    if (mla::launch_metadata(cache_seqlens, batch, num_parts, ovh, tile_meta, num_splits,
                             static_cast<hipStream_t>(stream)) != hipSuccess)
        return MLA_ERR_HIP;
    return MLA_OK;
}

mla_status_t mla_get_metadata_host(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int num_parts,
                                   int32_t* tile_meta, int32_t* num_splits) {
    const mla_status_t st = check_meta_args(cache_seqlens, batch, num_parts, tile_meta, num_splits);
    if (st != MLA_OK) return st;
    for (int b = 0; b < batch; ++b)
        if (cache_seqlens[b] < 0) return MLA_ERR_INVALID_ARG;
    mla::metadata_host(cache_seqlens, batch, num_parts, mla::meta_overhead_blocks((long long)h_q * s_q),
                       tile_meta, num_splits);
    return MLA_OK;
}

static mla_status_t decode_paged_impl(const void* q, const void* kcache, int64_t num_blocks,
                                      const int32_t* block_table, int max_blocks,
                                      const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                      float softmax_scale, int causal,
                                      const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                      void* workspace, size_t workspace_bytes,
                                      void* out, float* lse, void* stream, bool fp8,
                                      int d_qk = mla::kDqk, const float* sinks = nullptr,
                                      const void* kv_scale = nullptr, bool fp4 = false,
                                      mla::ScratchSource scratch = nullptr,
                                      const FusedParams* fused = nullptr) {
    if (!q || !kcache || !block_table || !cache_seqlens || !tile_meta || !num_splits || !out || !lse)
        return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_parts <= 0 || max_blocks <= 0 || num_blocks <= 0)
        return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
    if (fp4 && (!kv_scale || !aligned16(kv_scale))) return MLA_ERR_INVALID_ARG;
    if (fused && (!fused->weight || !fused->rope_cs || !fused->out_scale || !aligned16(fused->weight) ||
                  !aligned16(fused->rope_cs) || !std::isfinite(fused->eps) || fused->eps < 0.f))
        return MLA_ERR_INVALID_ARG;
    if ((long long)s_q * h_q > mla::kMaxRows) return MLA_ERR_UNSUPPORTED;
    if (batch > mla::kMaxBatchMeta) return MLA_ERR_UNSUPPORTED;
    const size_t need = mla_workspace_size(batch, s_q, h_q, num_parts);
    if (scratch) {
        // no caller workspace: the library's own fixed-size array, looked up only once every
        // host-side check has passed (a rejected call touches no device)
        const mla_status_t st = scratch(need, &workspace, &workspace_bytes);
        if (st != MLA_OK) return st;
    }
    if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (!workspace || !aligned16(workspace)) return MLA_ERR_INVALID_ARG;
    const int M = s_q * h_q;

    const long long slots = (long long)batch + num_parts;
    mla::AttnArgs a{};
    a.q = q;
    a.kv = kcache;
    a.block_table = block_table;
    a.seqlens = cache_seqlens;
    a.tile_meta = tile_meta;
    a.num_splits = num_splits;
    a.out = out;
    a.lse = lse;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          align256((size_t)slots * M * mla::kDv * sizeof(float)));
    a.batch = batch;
    a.s_q = s_q;
    a.h_q = h_q;
    a.M = M;
    a.max_blocks = max_blocks;
    a.causal = causal ? 1 : 0;
    a.num_parts = num_parts;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.kv_fp8 = fp8 ? 1 : 0;
    a.kv_fp4 = fp4 ? 1 : 0;
    a.kv_scale = kv_scale;
    a.kv_rows = num_blocks * mla::kPage;
    a.d_qk = d_qk;
    a.sinks = sinks;
    if (fused) {
        a.fused = 1;
        a.qn_weight = fused->weight;
        a.qn_eps = fused->eps;
        a.rope_cs = fused->rope_cs;
        a.out_scale = fused->out_scale;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mla::launch_decode(a, false, s) != hipSuccess) return MLA_ERR_HIP;
    const hipError_t e = fused ? mla::launch_combine_fused(a, s)
                               : mla::launch_combine(a.part_o, a.part_lse, num_splits, 0, batch, M, out, lse, s,
                                                     sinks, h_q, mla::decode_uses_wide(a, false));
    if (e != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

mla_status_t mla_decode_paged(const void* q, const void* kcache, int64_t num_blocks,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                              float softmax_scale, int causal,
                              const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                              void* workspace, size_t workspace_bytes,
                              void* out, float* lse, void* stream) {
    return decode_paged_impl(q, kcache, num_blocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                             softmax_scale, causal, tile_meta, num_splits, num_parts, workspace,
                             workspace_bytes, out, lse, stream, false);
}

}  // extern "C"

namespace mla {

mla_status_t decode_paged_scratch(const void* q, const void* kcache, int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  float softmax_scale, int causal,
                                  const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                  void* out, float* lse, void* stream, ScratchSource scratch) {
    return decode_paged_impl(q, kcache, num_blocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                             softmax_scale, causal, tile_meta, num_splits, num_parts, nullptr, 0, out, lse,
                             stream, false, kDqk, nullptr, nullptr, false, scratch);
}

}  // namespace mla

extern "C" {

mla_status_t mla_decode_paged_latent512(const void* q, const void* kcache, int64_t num_blocks,
                                       const int32_t* block_table, int max_blocks,
                                       const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                       float softmax_scale, int causal, const float* sinks,
                                       const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                       void* workspace, size_t workspace_bytes,
                                       void* out, float* lse, void* stream) {
    return decode_paged_impl(q, kcache, num_blocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                             softmax_scale, causal, tile_meta, num_splits, num_parts, workspace,
                             workspace_bytes, out, lse, stream, false, mla::kDv, sinks);
}

mla_status_t mla_decode_paged_fp4(const void* q, const void* kv_codes, const void* kv_scales, int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  float softmax_scale, int causal, const float* sinks,
                                  const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                  void* workspace, size_t workspace_bytes,
                                  void* out, float* lse, void* stream) {
    return decode_paged_impl(q, kv_codes, num_blocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                             softmax_scale, causal, tile_meta, num_splits, num_parts, workspace,
                             workspace_bytes, out, lse, stream, false, mla::kDv, sinks, kv_scales, true);
}

mla_status_t mla_decode_fused(const void* q, const void* kv_codes, const void* kv_scales, int64_t num_blocks,
                              const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                              int batch, int s_q, int h_q, float softmax_scale, int causal, const float* sinks,
                              const float* norm_weight, float norm_eps, const float* rope_cs,
                              const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                              void* workspace, size_t workspace_bytes,
                              void* out_fp8, float* out_scale, float* lse, void* stream) {
    const FusedParams f{norm_weight, norm_eps, rope_cs, out_scale};
    return decode_paged_impl(q, kv_codes, num_blocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                             softmax_scale, causal, tile_meta, num_splits, num_parts, workspace,
                             workspace_bytes, out_fp8, lse, stream, false, mla::kDv, sinks, kv_scales,
                             kv_scales != nullptr, nullptr, &f);
}

mla_status_t mla_decode_paged_fp8(const void* q, const void* kcache, int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks,
                                  const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                  float softmax_scale, int causal,
                                  const int32_t* tile_meta, const int32_t* num_splits, int num_parts,
                                  void* workspace, size_t workspace_bytes,
                                  void* out, float* lse, void* stream) {
    return decode_paged_impl(q, kcache, num_blocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                             softmax_scale, causal, tile_meta, num_splits, num_parts, workspace,
                             workspace_bytes, out, lse, stream, true);
}

mla_status_t mla_decode_sparse(const void* q, const void* kv, int64_t num_tokens,
                               const int32_t* indices, int topk,
                               int batch, int s_q, int h_q, float softmax_scale, int splits,
                               void* workspace, size_t workspace_bytes,
                               void* out, float* lse, void* stream) {
    if (!q || !kv || !indices || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || topk <= 0 || num_tokens <= 0 || splits < 0)
        return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
    if (h_q > mla::kMaxRows) return MLA_ERR_UNSUPPORTED;
    if ((long long)batch * s_q > (1LL << 24)) return MLA_ERR_UNSUPPORTED;
    int req = splits > 0 ? splits : sparse_auto_splits(batch, s_q, h_q, topk);
    const int max_splits = (topk + mla::kChunk - 1) / mla::kChunk;
    if (req > max_splits) req = max_splits;
    if (req < sparse_min_splits(topk)) req = sparse_min_splits(topk);
    const int eff = sparse_effective_splits(topk, req);
    const size_t need = mla_workspace_size_sparse(batch, s_q, h_q, topk, req);
    if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (eff > 1 && (!workspace || !aligned16(workspace))) return MLA_ERR_INVALID_ARG;

    const int groups = batch * s_q;
    mla::AttnArgs a{};
    a.q = q;
    a.kv = kv;
    a.indices = indices;
    a.out = out;
    a.lse = lse;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = eff > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                     align256((size_t)groups * eff * h_q * mla::kDv * sizeof(float)))
                         : nullptr;
    a.batch = groups;
    a.s_q = 1;
    a.h_q = h_q;
    a.M = h_q;
    a.topk = topk;
    a.kv_rows = num_tokens;
    a.d_qk = mla::kDqk;
    a.num_parts = eff;
    a.split_len = sparse_split_len(topk, req);
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mla::launch_decode(a, true, s) != hipSuccess) return MLA_ERR_HIP;
    if (eff > 1 && mla::launch_combine(a.part_o, a.part_lse, nullptr, eff, groups, h_q, out, lse, s) != hipSuccess)
        return MLA_ERR_HIP;
    return MLA_OK;
}

mla_status_t mla_sparse_prefill(const void* q, const void* kv, int64_t num_tokens,
                                const int32_t* indices, int topk, int s_q, int h_q,
                                float softmax_scale, int splits,
                                void* workspace, size_t workspace_bytes,
                                void* out, float* lse, void* stream) {
    // a prompt chunk is one "sequence" of s_q query tokens, each with its own index list
    return mla_decode_sparse(q, kv, num_tokens, indices, topk, 1, s_q, h_q, softmax_scale, splits,
                             workspace, workspace_bytes, out, lse, stream);
}

}  // extern "C"

namespace mla {

// Host twin of mla_metadata_kernel: the same integer partition, computed sequentially.
void metadata_host(const int32_t* seqlens, int batch, int num_parts, int ovh, int32_t* tile_meta,
                   int32_t* num_splits) {
    std::vector<long long> cpre(batch + 1, 0);
    std::vector<int> nb(batch, 0);
    for (int b = 0; b < batch; ++b) {
        const int L = seqlens[b];
        nb[b] = L > 0 ? (L + kPage - 1) / kPage : 0;
        cpre[b + 1] = cpre[b] + (nb[b] > 0 ? nb[b] + ovh : 0);
    }
    const long long total = cpre[batch];
    const long long payload = total > 0 ? (total + num_parts - 1) / num_parts : 1;
    num_splits[0] = 0;
    for (int b = 0; b < batch; ++b) {
        int sp = 0;
        if (nb[b] > 0) {
            const long long u0 = cpre[b] + ovh;
            sp = (int)((u0 + nb[b] - 1) / payload - u0 / payload + 1);
        }
        num_splits[b + 1] = num_splits[b] + sp;
    }
    for (int p = 0; p < num_parts; ++p) {
        int bb[2], blk[2];
        for (int e = 0; e < 2; ++e) {
            const long long u = (long long)(p + e) * payload;
            if (u >= total) {
                bb[e] = batch;
                blk[e] = 0;
                continue;
            }
            int b = 0;
            while (cpre[b + 1] <= u) ++b;
            bb[e] = b;
            const long long off = u - cpre[b] - ovh;
            blk[e] = off > 0 ? (int)off : 0;
        }
        int slot = 0;
        if (bb[0] < batch) {
            const long long first = (cpre[bb[0]] + ovh) / payload;
            slot = (p < first) ? 0 : (int)(num_splits[bb[0]] + (p - first));
        }
        int32_t* m = tile_meta + (size_t)p * kMetaInts;
        m[0] = bb[0]; m[1] = blk[0]; m[2] = bb[1]; m[3] = blk[1]; m[4] = slot;
        m[5] = 0; m[6] = 0; m[7] = 0;
    }
}

}  // namespace mla
