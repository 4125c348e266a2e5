// gfx950 (CDNA4) kernels for paged and sparse MLA decode.
//
// K0  mla_metadata_kernel   tile-scheduler metadata from device sequence lengths
// K1  mla_decode_kernel     gather -> Q.K^T (576) -> online softmax -> P.V (512) -> final or partial
//                           (paged bf16 cache, or sparse fp8 records through an index list)
// K2  mla_combine_kernel    LSE-weighted merge of split-KV partials
//
// The attention follows S = Q K^T, P = softmax(S), O = P V ("FlashMLA-ETAP: Efficient
// Transpose Attention Pipeline ...", section 방법론 / 핵심 메커니즘).  As in that paper's
// transposed form, each wave computes S^T = K Q^T with the KV tokens on the MFMA's M side,
// so 16 query rows fill a 16x16x32 bf16 MFMA without padding; the S^T accumulator layout is
// then directly the B operand of O^T = V^T P^T, and only V needs a transposed LDS read
// (ds_read_b64_tr_b16).  Everything else (chunking, LDS layout, XCD mapping, splits) is
// designed for CDNA4 here and not taken from the pages.
#include "mla_device.h"

namespace mla {

// --------------------------------------------------------------------------
// K1: decode kernel
// --------------------------------------------------------------------------
template <int NT, int RW, bool SPARSE>
struct DecodeCfg {
    static constexpr int TS = 4 / RW;                         // independent token streams
    static constexpr int ROWS_WAVE = 16 * NT;
    static constexpr int ROWS_WG = ROWS_WAVE * RW;
    static constexpr int LOADERS = 64 * RW;                   // threads loading one chunk
    // Loader shape.  Each wave of a stream owns rows rw, rw+RW, ...: one load instruction per
    // row puts lane L on 16-B granule L of that row (bf16: dims 8L..8L+7 of the first 512;
    // sparse fp8: granules 0..35 are the 576 codes and lane 36 fetches the granule holding
    // the fp32 scale).  bf16 rows also have granules 64..71 (the RoPE dims), spread over all
    // loaders of the stream.
    static constexpr int RA = kChunk / RW;                    // rows per loader wave
    static constexpr int RB = SPARSE ? 0 : (kChunk * 8) / LOADERS;
    static constexpr int BUF_BYTES = TS * kChunkBytes;
    static constexpr int MERGE_ACC_BYTES = (TS - 1) * RW * 32 * 64 * 16;   // one tile of acc per wave
    static constexpr int MERGE_ML_BYTES = (TS - 1) * RW * 64 * 8;
    static constexpr int MAIN_BYTES = BUF_BYTES > MERGE_ACC_BYTES + MERGE_ML_BYTES
                                          ? BUF_BYTES : MERGE_ACC_BYTES + MERGE_ML_BYTES;
    static constexpr int AUX_BYTES = SPARSE ? TS * kChunk * 8 : 0;          // per-row scale + valid flag
    static constexpr int LDS_BYTES = MAIN_BYTES + AUX_BYTES;
};

template <int NT, int RW, bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(const AttnArgs a) {
    using C = DecodeCfg<NT, RW, SPARSE>;
    constexpr int TS = C::TS;
    constexpr int RA = C::RA;
    constexpr int RB = C::RB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rw = wave % RW;
    const int ts = wave / RW;
    const int lt = rw * 64 + lane;             // loader index within this token stream
    const int g4 = lane >> 4;                  // lane group (0..3)
    const int l16 = lane & 15;

    char* buf = smem + ts * kChunkBytes;
    float* aux = reinterpret_cast<float*>(smem + C::MAIN_BYTES) + ts * kChunk;                // token scale
    int* auxok = reinterpret_cast<int*>(smem + C::MAIN_BYTES) + TS * kChunk + ts * kChunk;    // token used

    // ---- work item -> (part or sparse split, row group), XCD-aware -------------------------
    const int R = ceil_div(a.M, C::ROWS_WG);
    const int n_items = (SPARSE ? a.batch * a.num_parts : a.num_parts);
    int item, rg;
    xcd_item(blockIdx.x, n_items, R, item, rg);
    const int rbase = rg * C::ROWS_WG + rw * C::ROWS_WAVE;   // first row of this wave

    // LDS byte offsets that do not depend on the chunk.
    // K operand of S^T (ds_read_b128): row tt*16 + l16, granule ks*4 + g4; the XOR only touches
    // the low 3 granule bits, so for ks < 16 granule 8*(ks/2) + (4*(ks&1) + g4) sits at
    // kbase[tt][ks&1] + 128*(ks/2); ks = 16, 17 are the RoPE granules in region B.
    int kbase[2][2], kbaseB[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int row = tt * 16 + l16;
            kbase[tt][par] = lds_a(row, 4 * par + g4);
            kbaseB[tt][par] = lds_b(row, 4 * par + g4);
        }
    auto kaddr = [&](int tt, int ks) {
        return ks < 16 ? kbase[tt][ks & 1] + 128 * (ks >> 1) : kbaseB[tt][ks & 1];
    };
    // V^T operand (ds_read_b64_tr_b16): lane supplies token row 4*g4 + l16/4 (+16 for the upper
    // 16 tokens), dims 16*dt + 4*(l16&3) .. +3, i.e. granule 2*dt + ((l16&3)>>1), byte (l16&1)*8.
    // granule 8*(dt/4) + (2*(dt&3) + h) maps to vbase[half][dt&3] + 128*(dt/4).
    int vbase[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
            const int row = 4 * g4 + (l16 >> 2) + 16 * hf;
            vbase[hf][d4] = lds_a(row, 2 * d4 + ((l16 & 3) >> 1)) + (l16 & 1) * 8;
        }

    // per-segment state
    bf16x8 qf[NT][18];
    f4 acc[32][NT];
    float m_run[NT], l_run[NT];
    uint4 preA[RA];
    uint4 preB[RB > 0 ? RB : 1];
    int my_idx = -1;

    // ---- one segment: a contiguous token range of one sequence (or one sparse split) -------
    auto run_segment = [&](int grp, int t0, int t1, int L, bool final_out, int slot) {
        // Q fragments (B operand of S^T = K Q^T): lane holds row l16 of tile n, dims 8*g4 + 32*ks
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int r = rbase + 16 * n + l16;
            const char* qrow = static_cast<const char*>(a.q) + ((size_t)grp * a.M + (r < a.M ? r : 0)) * (kDqk * 2);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                uint4 v = *reinterpret_cast<const uint4*>(qrow + (ks * 32 + g4 * 8) * 2);
                if (r >= a.M) v = make_uint4(0, 0, 0, 0);
                qf[n][ks] = __builtin_bit_cast(bf16x8, v);
            }
            m_run[n] = -INFINITY;
            l_run[n] = 0.f;
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) acc[dt][n] = f4{0.f, 0.f, 0.f, 0.f};
        }
        const int nch = ceil_div(t1 - t0, kChunk);

        // causal limit per row of this lane (paged): query s sees t <= L - s_q + s
        int limit[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int r = rbase + 16 * n + l16;
            limit[n] = a.causal ? (L - a.s_q + r / a.h_q) : (L - 1);
        }

        // issue the global loads of chunk c into registers
        auto load_chunk = [&](int c, int jlo = 0, int jhi = C::RA) {
            if (c >= nch) return;
            const int tb = t0 + c * kChunk;
            const int nrows = min(kChunk, t1 - tb);
            if constexpr (!SPARSE && RW == 1) {
                // one wave per stream: copy HBM -> LDS directly (no registers).  Each instruction
                // writes 64 consecutive 16-B LDS slots; lane L of row r fetches the granule the
                // swizzle puts in slot L.  Rows past the segment end repeat its last row (finite
                // data, weight 0), so stale or NaN memory never reaches P.V.
                const int page = a.block_table[(size_t)grp * a.max_blocks + (tb >> 6)];
                const char* base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * kRowBytes;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int r = 0; r < kChunk; ++r) {
                    const int rr = min(r, nrows - 1);
                    dma16(base + rr * kRowBytes + ((lane ^ swz(r)) << 4), buf + r * kRowA);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int slot = j * 64 + lane;
                    const int row = slot >> 3;
                    const int rr = min(row, nrows - 1);
                    dma16(base + rr * kRowBytes + (64 + ((slot & 7) ^ swz(row))) * 16, buf + kRegionB + j * 1024);
                }
            } else if constexpr (!SPARSE) {
                // a chunk is 32 consecutive rows of one page: contiguous in HBM
                const int page = a.block_table[(size_t)grp * a.max_blocks + (tb >> 6)];
                const char* base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * kRowBytes;
#pragma unroll
                for (int j = 0; j < RA; ++j) {
                    const int row = rw + RW * j;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (row < nrows) v = load_nt(base + row * kRowBytes + lane * 16);
                    preA[j] = v;
                }
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    const int q = lt + C::LOADERS * j;
                    const int row = q >> 3, col = 64 + (q & 7);
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (row < nrows) v = load_nt(base + row * kRowBytes + col * 16);
                    preB[j] = v;
                }
            } else {
                // lanes 0..31 fetch the chunk's 32 indices; each row's index is then wave-uniform
                if (jlo == 0) {
                    my_idx = -1;
                    if (lane < nrows) my_idx = a.indices[(size_t)grp * a.topk + tb + lane];
                }
                const char* kvb = static_cast<const char*>(a.kv);
#pragma unroll
                for (int j = 0; j < RA; ++j) {
                    if (j < jlo || j >= jhi) continue;
                    const int row = rw + RW * j;
                    const int idx = __builtin_amdgcn_readlane(my_idx, row);
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (idx >= 0 && lane <= 36) v = load_nt(kvb + (size_t)idx * kRec + lane * 16);
                    preA[j] = v;
                }
            }
        };

        // write the prefetched chunk into this stream's LDS buffer (bf16, swizzled rows)
        auto store_chunk = [&](int jlo = 0, int jhi = C::RA) {
            if constexpr (!SPARSE && RW == 1) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the direct copies have landed
            } else if constexpr (!SPARSE) {
#pragma unroll
                for (int j = 0; j < RA; ++j) {
                    const int row = rw + RW * j;
                    *reinterpret_cast<uint4*>(buf + lds_a(row, lane)) = preA[j];
                }
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    const int q = lt + C::LOADERS * j;
                    *reinterpret_cast<uint4*>(buf + lds_b(q >> 3, q & 7)) = preB[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < RA; ++j) {
                    if (j < jlo || j >= jhi) continue;
                    const int row = rw + RW * j;
                    if (lane < 36) {
                        uint4 lo, hi;
                        fp8x16_to_bf16(preA[j], lo, hi);
                        const int o0 = lane < 32 ? lds_a(row, 2 * lane) : lds_b(row, 2 * lane - 64);
                        const int o1 = lane < 32 ? lds_a(row, 2 * lane + 1) : lds_b(row, 2 * lane - 63);
                        *reinterpret_cast<uint4*>(buf + o0) = lo;
                        *reinterpret_cast<uint4*>(buf + o1) = hi;
                    } else if (lane == 36) {
                        const int idx = __builtin_amdgcn_readlane(my_idx, row);
                        aux[row] = __builtin_bit_cast(float, preA[j].x);
                        auxok[row] = idx >= 0;
                    }
                }
            }
        };

        // compute on the chunk in LDS
        auto compute_chunk = [&](int c) {
            const int tb = t0 + c * kChunk;
            // S^T[token][row] = sum_k K[token][k] Q[row][k]
            f4 s[2][NT];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int n = 0; n < NT; ++n) s[tt][n] = f4{0.f, 0.f, 0.f, 0.f};
            // software-pipelined: the K fragments of step ks+1 are read while step ks multiplies;
            // the scheduling barriers keep the compiler from hoisting all 36 reads at once.
            bf16x8 kf[2][2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) kf[0][tt] = *reinterpret_cast<const bf16x8*>(buf + kaddr(tt, 0));
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                if (ks + 1 < 18) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
                        kf[(ks + 1) & 1][tt] = *reinterpret_cast<const bf16x8*>(buf + kaddr(tt, ks + 1));
                }
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int n = 0; n < NT; ++n) s[tt][n] = mfma16(kf[ks & 1][tt], qf[n][ks], s[tt][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // this lane's tokens are tt*16 + 4*g4 + i
            float tsc[2][4];
            bool tok_ok[2][4];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = tt * 16 + 4 * g4 + i;
                    if constexpr (SPARSE) {
                        tsc[tt][i] = aux[tok];
                        tok_ok[tt][i] = auxok[tok] != 0;
                    } else {
                        tsc[tt][i] = 1.f;
                        tok_ok[tt][i] = tb + tok < t1;
                    }
                }
            // scaled, masked scores and their per-row chunk maximum
            float x[NT][2][4];
            float mx[NT];
            bool grow = false;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                mx[n] = -INFINITY;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = tb + tt * 16 + 4 * g4 + i;
                        bool valid = tok_ok[tt][i];
                        if constexpr (!SPARSE) valid = valid && (t <= limit[n]);
                        const float f = SPARSE ? a.scale_log2 * tsc[tt][i] : a.scale_log2;
                        x[n][tt][i] = valid ? s[tt][n][i] * f : -INFINITY;
                        mx[n] = fmaxf(mx[n], x[n][tt][i]);
                    }
                mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 16));
                mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 32));
                grow = grow || (mx[n] > m_run[n] + kSlack);
            }
            // the softmax reference of a row only moves when the row's maximum outgrows it by
            // more than kSlack (log2 units); then the whole wave rescales once.
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const float m_new = fmaxf(m_run[n], mx[n]);
                    const float alpha = exp2_fast(m_run[n] - (m_new == -INFINITY ? 0.f : m_new));
                    l_run[n] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 32; ++dt) acc[dt][n] *= alpha;
                    m_run[n] = m_new;
                }
            }
            bf16x8 pT[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float m_use = (m_run[n] == -INFINITY) ? 0.f : m_run[n];
                float p[2][4];
                float psum = 0.f;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[tt][i] = exp2_fast(x[n][tt][i] - m_use);
                        psum += p[tt][i];
                        if constexpr (SPARSE) p[tt][i] *= tsc[tt][i];
                    }
                l_run[n] += psum;
                // B operand of O^T = V^T P^T: k index 8*g4 + j <-> token j<4 ? 4*g4+j : 16+4*g4+(j-4)
                const uint4 pk = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                            pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
                pT[n] = __builtin_bit_cast(bf16x8, pk);
            }
            // O^T[d][row] += sum_token V[token][d] P[row][token]; V^T fragments of dt+1 are read
            // (transposing LDS reads) while dt multiplies.
            auto read_vt = [&](int dt) {
                const int off = 128 * (dt >> 2);
                const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4v*)(buf + vbase[0][dt & 3] + off));
                const short4v v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4v*)(buf + vbase[1][dt & 3] + off));
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            bf16x8 vf[2];
            vf[0] = read_vt(0);
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) {
                if (dt + 1 < 32) vf[(dt + 1) & 1] = read_vt(dt + 1);
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[dt][n] = mfma16(vf[dt & 1], pT[n], acc[dt][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // ---- chunk loop: all waves run the same trip count (barriers inside) ----
        // With one wave per stream (RW == 1) the stream's LDS buffer is private to that wave: it
        // orders its own LDS writes and reads, and the 4 waves of the block run unsynchronised,
        // so one wave's loads overlap another's compute.  With several waves per stream the
        // chunk is shared and the next chunk is prefetched into registers during compute.
        auto stream_sync = [&]() {
            if constexpr (RW == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            else __syncthreads();
        };
        constexpr bool kPrefetch = RW > 1;
        if constexpr (kPrefetch) load_chunk(ts);
        for (int cb = 0; cb < nch; cb += TS) {
            const int c = cb + ts;
            stream_sync();               // previous chunk's LDS reads are done
            if constexpr (SPARSE && !kPrefetch) {
                // gathered rows go through registers: two halves keep the register count down
                if (c < nch) {
                    load_chunk(c, 0, RA / 2);
                    store_chunk(0, RA / 2);
                    load_chunk(c, RA / 2, RA);
                    store_chunk(RA / 2, RA);
                }
            } else {
                if constexpr (!kPrefetch) load_chunk(c);
                if (kPrefetch || c < nch) store_chunk();
            }
            stream_sync();               // chunk visible to the stream's waves
            if constexpr (kPrefetch) load_chunk(c + TS);   // next chunk in flight during compute
            if (c < nch) compute_chunk(c);
        }

        // ---- finish: row sums, merge token streams, write ----
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            l_run[n] += __shfl_xor(l_run[n], 16);
            l_run[n] += __shfl_xor(l_run[n], 32);
        }
        if constexpr (TS > 1) {
            f4* macc = reinterpret_cast<f4*>(smem);
            float* mml = reinterpret_cast<float*>(smem + C::MERGE_ACC_BYTES);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                __syncthreads();
                if (ts > 0) {
                    const int w = (ts - 1) * RW + rw;
#pragma unroll
                    for (int dt = 0; dt < 32; ++dt) macc[(w * 32 + dt) * 64 + lane] = acc[dt][n];
                    mml[(w * 64 + lane) * 2 + 0] = m_run[n];
                    mml[(w * 64 + lane) * 2 + 1] = l_run[n];
                }
                __syncthreads();
                if (ts == 0) {
                    float mk[TS], lk[TS];
                    mk[0] = m_run[n];
                    lk[0] = l_run[n];
                    float m_new = mk[0];
#pragma unroll
                    for (int k = 1; k < TS; ++k) {
                        const int w = (k - 1) * RW + rw;
                        mk[k] = mml[(w * 64 + lane) * 2 + 0];
                        lk[k] = mml[(w * 64 + lane) * 2 + 1];
                        m_new = fmaxf(m_new, mk[k]);
                    }
                    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                    float al[TS];
                    float l_new = 0.f;
#pragma unroll
                    for (int k = 0; k < TS; ++k) {
                        al[k] = exp2_fast(mk[k] - m_use);
                        l_new += al[k] * lk[k];
                    }
#pragma unroll
                    for (int dt = 0; dt < 32; ++dt) {
                        f4 v = acc[dt][n] * al[0];
#pragma unroll
                        for (int k = 1; k < TS; ++k) {
                            const int w = (k - 1) * RW + rw;
                            v += macc[(w * 32 + dt) * 64 + lane] * al[k];
                        }
                        acc[dt][n] = v;
                    }
                    m_run[n] = m_new;
                    l_run[n] = l_new;
                }
            }
        }
        if (ts == 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int r = rbase + 16 * n + l16;
                const float l = l_run[n];
                const float inv = l > 0.f ? 1.f / l : 0.f;
                const float lse_v = l > 0.f ? (m_run[n] + __log2f(l)) * kLn2 : -INFINITY;
                if (r < a.M) {
                    if (final_out) {
                        __bf16* orow = static_cast<__bf16*>(a.out) + ((size_t)grp * a.M + r) * kDv + 4 * g4;
#pragma unroll
                        for (int dt = 0; dt < 32; ++dt) {
                            const f4 v = acc[dt][n] * inv;
                            const uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                            *reinterpret_cast<uint2*>(orow + dt * 16) = pk;
                        }
                        if (g4 == 0) a.lse[(size_t)grp * a.M + r] = lse_v;
                    } else {
                        float* prow = a.part_o + ((size_t)slot * a.M + r) * kDv + 4 * g4;
#pragma unroll
                        for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<f4*>(prow + dt * 16) = acc[dt][n] * inv;
                        if (g4 == 0) a.part_lse[(size_t)slot * a.M + r] = lse_v;
                    }
                }
            }
        }
    };

    if constexpr (!SPARSE) {
        const int* meta = a.tile_meta + (size_t)item * kMetaInts;
        const int b0 = meta[0], blk0 = meta[1], b1 = meta[2], blk1 = meta[3], slot0 = meta[4];
        for (int bb = b0; bb <= b1 && bb < a.batch; ++bb) {
            const int L = a.seqlens[bb];
            const int nb = ceil_div(L, kPage);
            const int lo = (bb == b0) ? blk0 : 0;
            const int hi = (bb == b1) ? blk1 : nb;
            if (lo >= hi) continue;
            const int nsp = a.num_splits[bb + 1] - a.num_splits[bb];
            const int slot = (bb == b0) ? slot0 : a.num_splits[bb];
            run_segment(bb, lo * kPage, min(hi * kPage, L), L, nsp == 1, slot);
            __syncthreads();
        }
    } else {
        const int grp = item / a.num_parts;          // query token (b*s_q + s)
        const int split = item % a.num_parts;
        const int e0 = split * a.split_len;
        const int e1 = min(e0 + a.split_len, a.topk);
        if (e0 < e1)
            run_segment(grp, e0, e1, 0, a.num_parts == 1, grp * a.num_parts + split);
    }
}

// --------------------------------------------------------------------------
// K1m: paged decode for one 16-row tile (s_q * h_q <= 16), the memory-bound shape.
// Four independent token streams per block (one per wave, one wave per SIMD).  Each stream
// double-buffers 16-token chunks (18 KB) that go HBM -> LDS by direct copies, so one chunk is
// always in flight while the previous one is multiplied; the streams merge at the end.
// Region A (dims 0..511) keeps a token's 1 KB unswizzled at a 1056-byte stride: the 16 tokens x
// 64 B of a K read and the transposing V^T reads fall on distinct banks (the 1024-byte stride
// with the chunk kernels' XOR swizzle left 47% of this kernel's LDS cycles in bank conflicts).
// --------------------------------------------------------------------------
constexpr int kMChunk = 16;
constexpr int kMRowA = 1056;                                 // region A row stride (1 KB + 32 B)
constexpr int kMBuf = kMChunk * kMRowA + kMChunk * 128;     // region A then region B
constexpr int kMRegionB = kMChunk * kMRowA;
constexpr int kMDmaOps = kMChunk + 2;                        // copy instructions per chunk and wave

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_m16_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[4 * 2 * kMBuf];   // 148 KB
    __shared__ int s_pages[4][64];                                       // per-wave page window
    const int lane = threadIdx.x & 63;
    const int ts = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);     // stream = wave
    const int g4 = lane >> 4, l16 = lane & 15;
    char* bufs = smem + ts * 2 * kMBuf;
    const int item = blockIdx.x;

    // K fragment (A operand of S^T): token row l16, granule 4*ks + g4
    int kA[2], kB[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        kA[par] = l16 * kMRowA + ((4 * par + g4) << 4);
        kB[par] = kMRegionB + l16 * 128 + (((4 * par + g4) ^ swz(l16)) << 4);
    }
    // V^T fragment (A operand of O^T, 16x16x16): tokens 4*g4..+3, dims 16*dt + l16 via one
    // transposing read; lane supplies row 4*g4 + l16/4, dims 16*dt + 4*(l16&3)..+3
    int vb[4];
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
        const int row = 4 * g4 + (l16 >> 2);
        vb[d4] = row * kMRowA + ((2 * d4 + ((l16 & 3) >> 1)) << 4) + (l16 & 1) * 8;
    }

    bf16x8 qf[18];
    f4 acc[32];
    float m_run, l_run;

    // Q of a segment: the workgroup copies its 16 rows (18 KB, rows past M repeat row 0) into
    // wave 0's second buffer, each wave a quarter; every wave then reads its fragments from there
    char* const qs = smem + kMBuf;
    auto copy_q = [&](int grp) {
        const char* qg = static_cast<const char*>(a.q) + (size_t)grp * a.M * (kDqk * 2);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int j = ts + 4 * i;
            if (j < 18) {
                const unsigned e = 1024 * j + 16 * lane;
                const unsigned row = e / (kDqk * 2), col = e % (kDqk * 2);
                dma16_s_shared(qg, ((int)row < a.M ? row : 0) * (kDqk * 2) + col, qs + 1024 * j);
            }
        }
    };

    // win0: lane i holds the block-table entry of page t0/64 + i (loaded by the caller)
    auto run_segment = [&](int grp, int t0, int t1, int L, bool final_out, int slot, int win0) {
        const int r = l16;
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) acc[dt] = f4{0.f, 0.f, 0.f, 0.f};
        const int limit = a.causal ? (L - a.s_q + r / a.h_q) : (L - 1);
        const int nch = ceil_div(t1 - t0, kMChunk);

        // Wave ts handles chunks c = ts + 4k: rows 16*ts..16*ts+15 of page lo + k.  The page
        // numbers come 64 at a time into a per-wave LDS window (the first from the caller), so
        // looking one up never waits on the vector-memory counter (which also counts the
        // in-flight KV copies).
        const int lo_page = t0 >> 6;
        int bt_base = 0;
        s_pages[ts][lane] = win0;
        auto page_of = [&](int k) {
            if (k - bt_base >= 64 || k < bt_base) {
                bt_base = k;
                const int np = ceil_div(t1, kPage) - lo_page;
                const int v = (lane < np - k) ? a.block_table[(size_t)grp * a.max_blocks + lo_page + k + lane] : 0;
                s_pages[ts][lane] = v;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            return __builtin_amdgcn_readfirstlane(s_pages[ts][k - bt_base]);
        };
        // copy chunk c = ts + 4k (16 rows of one page, contiguous in HBM) into buffer b
        auto issue = [&](int k, int b) {
            const int c = ts + 4 * k;
            const int tb = t0 + c * kMChunk;
            const int nrows = min(kMChunk, t1 - tb);
            const int page = page_of(k);
            const char* base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * kRowBytes;
            char* dst = bufs + b * kMBuf;
#pragma unroll
            for (int row = 0; row < kMChunk; ++row) {
                const int rr = min(row, nrows - 1);   // rows past the end repeat the last row (weight 0)
                dma16(base + rr * kRowBytes + (lane << 4), dst + row * kMRowA);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int sl = j * 64 + lane;
                const int row = sl >> 3;
                const int rr = min(row, nrows - 1);
                dma16(base + rr * kRowBytes + (64 + ((sl & 7) ^ swz(row))) * 16, dst + kMRegionB + j * 1024);
            }
        };

        if (ts < nch) {
            issue(0, 0);
        }
        // Q: the caller waited for this wave's copies; the barrier covers the other waves', the
        // second one every wave's reads before wave 0 refills the buffer
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            uint4 v = *reinterpret_cast<const uint4*>(qs + r * (kDqk * 2) + (ks * 32 + g4 * 8) * 2);
            if (r >= a.M) v = make_uint4(0, 0, 0, 0);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
        int k = 0;
        for (int c = ts; c < nch; c += 4, ++k) {
            const char* buf = bufs + (k & 1) * kMBuf;
            if (c + 4 < nch) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of the other buffer done
                issue(k + 1, (k + 1) & 1);
                asm volatile("s_waitcnt vmcnt(18)" ::: "memory");    // chunk c landed, c+4 in flight
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            const int tb = t0 + c * kMChunk;
            // S^T[token][row] over 576 dims: two accumulators (even / odd k steps) break the chain.
            // K fragments are read four MFMA steps ahead and V^T fragments six, with the schedule
            // pinned to (read, MFMA) pairs so that the one wave per SIMD keeps LDS reads in flight.
            f4 sacc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
            auto kread = [&](int ks) {
                const int off = ks < 16 ? kA[ks & 1] + 128 * (ks >> 1) : kB[ks & 1];
                return *reinterpret_cast<const bf16x8*>(buf + off);
            };
            bf16x8 kw[18];
#pragma unroll
            for (int i = 0; i < 4; ++i) kw[i] = kread(i);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                if (ks + 4 < 18) kw[ks + 4] = kread(ks + 4);
                sacc[ks & 1] = mfma16(kw[ks], qf[ks], sacc[ks & 1]);
                if (ks + 4 < 18) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            auto vread = [&](int dt) {
                return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vb[dt & 3] + 128 * (dt >> 2)));
            };
            short4v vw[32];
#pragma unroll
            for (int dt = 0; dt < 6; ++dt) vw[dt] = vread(dt);
            const f4 sv = sacc[0] + sacc[1];
            float x[4];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tb + 4 * g4 + i;
                x[i] = (t < t1 && t <= limit) ? sv[i] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, x[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = exp2_fast(m_run - (m_new == -INFINITY ? 0.f : m_new));
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < 32; ++dt) acc[dt] *= alpha;
                m_run = m_new;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = exp2_fast(x[i] - m_use);
                l_run += p[i];
            }
            // P^T (B operand, k = tokens 4*g4..+3, n = row l16) is the S^T accumulator layout
            const short4v pT = __builtin_bit_cast(short4v, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) {
                if (dt + 6 < 32) vw[dt + 6] = vread(dt + 6);
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vw[dt], pT, acc[dt], 0, 0, 0);
                if (dt + 6 < 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            }
        }

        // row sums, then the 4 streams merge through LDS: every wave stores its accumulators,
        // and wave ts merges and writes value tiles 8*ts..8*ts+7 of all four
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        f4* macc = reinterpret_cast<f4*>(smem);                                 // [stream][tile][lane]
        float* mml = reinterpret_cast<float*>(smem + 4 * 32 * 64 * 16);        // [stream][lane][m, l]
        __syncthreads();
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) macc[(ts * 32 + dt) * 64 + lane] = acc[dt];
        mml[(ts * 64 + lane) * 2 + 0] = m_run;
        mml[(ts * 64 + lane) * 2 + 1] = l_run;
        __syncthreads();
        {
            float mk[4], lk[4];
            mk[0] = mml[lane * 2 + 0];
            lk[0] = mml[lane * 2 + 1];
            float m_new = mk[0];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                mk[w] = mml[(w * 64 + lane) * 2 + 0];
                lk[w] = mml[(w * 64 + lane) * 2 + 1];
                m_new = fmaxf(m_new, mk[w]);
            }
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            float al[4], l_new = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                al[w] = exp2_fast(mk[w] - m_use);
                l_new += al[w] * lk[w];
            }
            const float inv = l_new > 0.f ? 1.f / l_new : 0.f;
            const float lse_v = l_new > 0.f ? (m_new + __log2f(l_new)) * kLn2 : -INFINITY;
            if (r < a.M) {
                if (final_out) {
                    __bf16* orow = static_cast<__bf16*>(a.out) + ((size_t)grp * a.M + r) * kDv + 4 * g4;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int dt = 8 * ts + j;
                        f4 v = macc[dt * 64 + lane] * al[0];
#pragma unroll
                        for (int w = 1; w < 4; ++w) v += macc[(w * 32 + dt) * 64 + lane] * al[w];
                        v *= inv;
                        *reinterpret_cast<uint2*>(orow + dt * 16) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
                    if (ts == 0 && g4 == 0) a.lse[(size_t)grp * a.M + r] = lse_v;
                } else {
                    float* prow = a.part_o + ((size_t)slot * a.M + r) * kDv + 4 * g4;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int dt = 8 * ts + j;
                        f4 v = macc[dt * 64 + lane] * al[0];
#pragma unroll
                        for (int w = 1; w < 4; ++w) v += macc[(w * 32 + dt) * 64 + lane] * al[w];
                        *reinterpret_cast<f4*>(prow + dt * 16) = v * inv;
                    }
                    if (ts == 0 && g4 == 0) a.part_lse[(size_t)slot * a.M + r] = lse_v;
                }
            }
        }
        __syncthreads();
    };

    const int* meta = a.tile_meta + (size_t)item * kMetaInts;
    const int b0 = meta[0], blk0 = meta[1], b1 = meta[2], blk1 = meta[3], slot0 = meta[4];
    for (int bb = b0; bb <= b1 && bb < a.batch; ++bb) {
        // A segment's first loads go out together, one memory round trip before its first KV
        // copy: the copy of Q, the first 64 entries of its block-table row from page lo (in
        // bounds of the row; entries past the sequence are never used), its length and split
        // count.  All of them are waited for (the empty asm reads the window) before the KV
        // copies start, so no load the compiler tracks is pending behind a copy.  (The copy of Q
        // goes first: the compiler's waits on the later loads then cover it.)
        copy_q(bb);
        const int lo = (bb == b0) ? blk0 : 0;
        const int win0 = (lane < a.max_blocks - lo) ? a.block_table[(size_t)bb * a.max_blocks + lo + lane] : 0;
        const int L = a.seqlens[bb];
        const int ns0 = a.num_splits[bb], ns1 = a.num_splits[bb + 1];
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("" ::"v"(win0));
        const int hi = (bb == b1) ? blk1 : ceil_div(L, kPage);
        if (lo >= hi) continue;
        run_segment(bb, lo * kPage, min(hi * kPage, L), L, ns1 - ns0 == 1, (bb == b0) ? slot0 : ns0, win0);
    }
}

// --------------------------------------------------------------------------
// K2: combine split-KV partials (one wave per output row, 8 dims per lane)
// --------------------------------------------------------------------------
// splits loaded together per round trip: 4 for the bf16 partials (at most a few splits per row),
// 8 for the fp32 ones (the 16-row kernel splits long sequences into many parts)
template <bool BF16>
constexpr int combine_group() { return BF16 ? 4 : 8; }
// dims d .. d+7 of a partial O row: fp32 (two 16-byte loads), or bf16 (one 16-byte load; BF16:
// the one-wave-per-SIMD kernel's 128-row groups)
template <bool BF16>
__device__ __forceinline__ void load_part8(const float* part_o, size_t row, int d, f4& lo, f4& hi) {
    if constexpr (BF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(part_o) + (row * kDv + d) * 2);
        lo = f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
        hi = f4{__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u),
                __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)};
    } else {
        lo = *reinterpret_cast<const f4*>(part_o + row * kDv + d);
        hi = *reinterpret_cast<const f4*>(part_o + row * kDv + d + 4);
    }
}

// The LSE-weighted merge of one row's n partials (slots base .. base+n-1) for the lane's dims
// d .. d+7: o[0..1] = sum_i exp(lse_i - mu) O_i / wsum, with an attention sink sk as one more
// term of the denominator (LSE = the sink, no value).  The splits go in groups of G whose LSEs
// and values are loaded together (one memory round trip per group); mu is the running
// maximum, and a group that raises it rescales what the earlier groups summed.
template <bool BF16, int NV = 2>
__device__ __forceinline__ void merge_row(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                          int base, int n, int rows, int r, int d, float sk,
                                          f4 (&o)[NV], float& mu, float& wsum) {
    static_assert(NV == 2 || !BF16, "bf16 partials: 8 dims per lane");
    mu = sk;
    wsum = sk != -INFINITY ? 1.f : 0.f;
#pragma unroll
    for (int q = 0; q < NV; ++q) o[q] = f4{0.f, 0.f, 0.f, 0.f};
    constexpr int G = combine_group<BF16>();
    for (int i0 = 0; i0 < n; i0 += G) {
        float li[G];
        f4 v[G][NV];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            // (n is the same for the whole wave: the branch does not diverge)
            li[j] = -INFINITY;
#pragma unroll
            for (int q = 0; q < NV; ++q) v[j][q] = f4{0.f, 0.f, 0.f, 0.f};
            if (i0 + j < n) {
                const size_t i = (size_t)(base + i0 + j) * rows + r;
                li[j] = part_lse[i];
                if constexpr (NV == 2) load_part8<BF16>(part_o, i, d, v[j][0], v[j][1]);
                else v[j][0] = *reinterpret_cast<const f4*>(part_o + i * kDv + d);
            }
        }
        float mg = mu;
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (i0 + j < n) mg = fmaxf(mg, li[j]);
        if (mg == -INFINITY) continue;                          // nothing finite so far
        const float sc = mu == -INFINITY ? 0.f : expf(mu - mg);  // mu <= mg
        wsum *= sc;
#pragma unroll
        for (int q = 0; q < NV; ++q) o[q] *= sc;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (i0 + j < n && li[j] != -INFINITY) {
                const float w = expf(li[j] - mg);
                wsum += w;
#pragma unroll
                for (int q = 0; q < NV; ++q) o[q] += v[j][q] * w;
            }
        }
        mu = mg;
    }
    if (mu != -INFINITY) {
        const float iw = 1.f / wsum;
#pragma unroll
        for (int q = 0; q < NV; ++q) o[q] *= iw;
    }
}

// BF16 partials: one wave per row, 8 dims per lane; fp32 partials: two waves per row (the
// value halves), 4 dims per lane, so that a row with many splits has twice the loads in flight
template <bool BF16>
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const int32_t* __restrict__ prefix,
                                                          int uniform_splits, int rows,
                                                          __bf16* __restrict__ out, float* __restrict__ lse,
                                                          const float* __restrict__ sinks, int h_q) {
    constexpr int WPR = BF16 ? 1 : 2;                 // waves per row
    const int grp = blockIdx.x;
    const int w = threadIdx.x >> 6;
    const int r = blockIdx.y * (4 / WPR) + w / WPR;
    const int half = w % WPR;
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    int base, n;
    if (prefix) {
        base = prefix[grp];
        n = prefix[grp + 1] - base;
    } else {
        base = grp * uniform_splits;
        n = uniform_splits;
    }
    if (n == 1) return;   // the decode kernel wrote this row directly
    const float sk = sinks ? sinks[r % h_q] : -INFINITY;
    float mu, wsum;
    if constexpr (BF16) {
        f4 o[2];
        merge_row<BF16>(part_o, part_lse, base, n, rows, r, 8 * lane, sk, o, mu, wsum);
        const uint4 pk = make_uint4(pack_bf16x2(o[0][0], o[0][1]), pack_bf16x2(o[0][2], o[0][3]),
                                    pack_bf16x2(o[1][0], o[1][1]), pack_bf16x2(o[1][2], o[1][3]));
        *reinterpret_cast<uint4*>(out + ((size_t)grp * rows + r) * kDv + 8 * lane) = pk;
    } else {
        f4 o[1];
        const int d = (kDv / 2) * half + 4 * lane;
        merge_row<BF16, 1>(part_o, part_lse, base, n, rows, r, d, sk, o, mu, wsum);
        *reinterpret_cast<uint2*>(out + ((size_t)grp * rows + r) * kDv + d) =
            make_uint2(pack_bf16x2(o[0][0], o[0][1]), pack_bf16x2(o[0][2], o[0][3]));
    }
    if (lane == 0 && half == 0) lse[(size_t)grp * rows + r] = (mu == -INFINITY) ? -INFINITY : mu + logf(wsum);
}

// --------------------------------------------------------------------------
// K0: tile-scheduler metadata (one workgroup; integer only, same partition as the host twin)
// --------------------------------------------------------------------------
constexpr int kMetaThreads = 256;

// exclusive scan of v over the workgroup's threads, and the workgroup total: a shuffle scan in
// each wave, then one over the wave totals (tmp holds kMetaThreads / 64 ints)
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
    constexpr int kWavesMeta = kMetaThreads / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) tmp[w] = x;
    __syncthreads();
    if (w == 0) {
        int s = lane < kWavesMeta ? tmp[lane] : 0;
#pragma unroll
        for (int off = 1; off < kWavesMeta; off <<= 1) {
            const int y = __shfl_up(s, off);
            if (lane >= off) s += y;
        }
        if (lane < kWavesMeta) tmp[lane] = s;
    }
    __syncthreads();
    const int before = w > 0 ? tmp[w - 1] : 0;
    total = tmp[kWavesMeta - 1];
    __syncthreads();
    return before + x - v;
}

__global__ __launch_bounds__(kMetaThreads) void mla_metadata_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                                    int num_parts, int ovh,
                                                                    int32_t* __restrict__ tile_meta,
                                                                    int32_t* __restrict__ num_splits) {
    __shared__ int cpre[kMaxBatchMeta + 1];   // cost prefix C_b
    __shared__ int spre[kMaxBatchMeta + 1];   // split prefix
    __shared__ int tmp[kMetaThreads / 64];
    __shared__ int s_payload;
    const int t = threadIdx.x;
    // cost prefix
    int carry = 0;
    for (int b0 = 0; b0 < batch; b0 += kMetaThreads) {
        const int b = b0 + t;
        int cost = 0;
        if (b < batch) {
            const int L = seqlens[b];
            const int nb = L > 0 ? (L + kPage - 1) / kPage : 0;
            cost = nb > 0 ? nb + ovh : 0;
        }
        int tot;
        const int ex = block_excl_scan(cost, tmp, tot);
        if (b < batch) cpre[b] = carry + ex;
        carry += tot;
    }
    if (t == 0) cpre[batch] = carry;
    const int total = carry;
    if (t == 0) s_payload = total > 0 ? (total + num_parts - 1) / num_parts : 1;
    __syncthreads();
    const int payload = s_payload;
    // splits per sequence and their prefix
    carry = 0;
    for (int b0 = 0; b0 < batch; b0 += kMetaThreads) {
        const int b = b0 + t;
        int sp = 0;
        if (b < batch) {
            // the sequence's blocks from its cost (the lengths are not read a second time)
            const int cost = cpre[b + 1] - cpre[b];
            const int nb = cost > 0 ? cost - ovh : 0;
            if (nb > 0) {
                const int u0 = cpre[b] + ovh;
                sp = (u0 + nb - 1) / payload - u0 / payload + 1;
            }
        }
        int tot;
        const int ex = block_excl_scan(sp, tmp, tot);
        if (b < batch) spre[b] = carry + ex;
        carry += tot;
    }
    if (t == 0) spre[batch] = carry;
    __syncthreads();
    for (int b = t; b <= batch; b += kMetaThreads) num_splits[b] = spre[b];
    // parts
    for (int p = t; p < num_parts; p += kMetaThreads) {
        int bb[2], blk[2];
        for (int e = 0; e < 2; ++e) {
            const long long u = (long long)(p + e) * payload;
            if (u >= total) {
                bb[e] = batch;
                blk[e] = 0;
                continue;
            }
            // b = number of sequences whose cost range ends at or before u
            int lo = 0, hi = batch;   // find first b with cpre[b+1] > u
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (cpre[mid + 1] <= u) lo = mid + 1; else hi = mid;
            }
            bb[e] = lo;
            const int off = (int)(u - cpre[lo]) - ovh;
            blk[e] = off > 0 ? off : 0;
        }
        int slot = 0;
        if (bb[0] < batch) {
            const int first = (cpre[bb[0]] + ovh) / payload;
            slot = spre[bb[0]] + (p - first);
            if (p < first) slot = 0;
        }
        int32_t* m = tile_meta + (size_t)p * kMetaInts;
        m[0] = bb[0]; m[1] = blk[0]; m[2] = bb[1]; m[3] = blk[1]; m[4] = slot;
        m[5] = 0; m[6] = 0; m[7] = 0;
    }
}

// --------------------------------------------------------------------------
// Launchers
// --------------------------------------------------------------------------
Tiling choose_tiling(int rows) {
    // <= 16 rows: one 16-row tile per workgroup (mla_decode_m16_kernel, or the 16-row sparse
    // kernel); up to 32 rows: one wave pair of mla_decode_big_kernel; more: 64-row workgroups
    // of mla_decode_rows_kernel.
    Tiling t;
    if (rows <= 16) {
        t.nt = 1;
        t.rw = 1;
    } else {
        t.nt = 2;
        t.rw = big_pairs(rows);
    }
    t.rows_wg = 16 * t.nt * t.rw;
    t.row_groups = (rows + t.rows_wg - 1) / t.rows_wg;
    return t;
}

hipError_t launch_metadata(const int32_t* seqlens, int batch, int num_parts, int overhead,
                           int32_t* tile_meta, int32_t* num_splits, hipStream_t stream) {
    hipLaunchKernelGGL(mla_metadata_kernel, dim3(1), dim3(kMetaThreads), 0, stream,
                       seqlens, batch, num_parts, overhead, tile_meta, num_splits);
    return hipGetLastError();
}

template <int NT, int RW, bool SPARSE>
static hipError_t launch_decode_t(const AttnArgs& a, int items, int R, hipStream_t stream) {
    hipLaunchKernelGGL((mla_decode_kernel<NT, RW, SPARSE>), dim3(items * R), dim3(256), 0, stream, a);
    return hipGetLastError();
}

bool decode_uses_wide(const AttnArgs& a, bool sparse) {
    // the fused decode, whatever the rows; bf16 and FP4 pages with more than 64 rows (576-wide
    // bf16 rows need a positive scale, which the kernel applies in the exponent)
    if (sparse || a.kv_fp8) return false;
    return a.fused || (a.M > kWideMinRows && (a.kv_fp4 || a.d_qk == kDv || a.scale_log2 > 0.f));
}

hipError_t launch_decode(const AttnArgs& a, bool sparse, hipStream_t stream) {
    const Tiling t = choose_tiling(a.M);
    if (decode_uses_wide(a, sparse)) return launch_decode_wide(a, stream);
    // 512-wide rows (K and V): the row-split kernel, whatever the rows and the scale
    if (!sparse && a.d_qk == kDv) return launch_decode_rows(a, false, stream);
    if (!sparse && a.kv_fp8) {
        // fp8 pages: the 16-row streaming kernel, or the row-split kernel's fp8 gathers
        if (a.M <= 16) return launch_decode_m16_fp8(a, stream);
        return launch_decode_rows(a, false, stream);
    }
    if (!sparse && a.M <= 16) {
        hipLaunchKernelGGL(mla_decode_m16_kernel, dim3(a.num_parts), dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    // the row-split kernel applies the scale in the exponent, which needs it positive
    if (!sparse && a.M > 32 && a.scale_log2 > 0.f) return launch_decode_rows(a, false, stream);
    // sparse, more than 32 heads: the row-split kernel
    if (sparse && a.M > 32) return launch_decode_rows(a, true, stream);
    if (a.M > 16) return launch_decode_big(a, sparse, stream);
    const int items = sparse ? a.batch * a.num_parts : a.num_parts;
    const int R = t.row_groups;
#define MLA_DISPATCH(NT_, RW_)                                                     \
    if (t.nt == NT_ && t.rw == RW_)                                                \
        return sparse ? launch_decode_t<NT_, RW_, true>(a, items, R, stream)       \
                      : launch_decode_t<NT_, RW_, false>(a, items, R, stream);
    MLA_DISPATCH(1, 1)
#undef MLA_DISPATCH
    return hipErrorInvalidValue;
}

// The combine of the fused decode: one wave per output row of a split sequence.  The LSE-weighted
// merge of the row's partials (as mla_combine_kernel), then the conjugate rotation of dims
// 448..511 by the query token's angles and the FP8 cast with one scale per row (amax / 448).
// Lane l holds dims 8l .. 8l+7.
__global__ __launch_bounds__(256) void mla_combine_fused_kernel(const AttnArgs a) {
    const int grp = blockIdx.x;
    const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int rows = a.M;
    if (r >= rows) return;
    const int base = a.num_splits[grp];
    const int n = a.num_splits[grp + 1] - base;
    if (n == 1) return;   // the decode kernel wrote this row directly
    const float sk = a.sinks ? a.sinks[r % a.h_q] : -INFINITY;
    f4 o[2];
    float mu, wsum;
    // (the fused decode runs on the one-wave-per-SIMD kernel: bf16 partials)
    merge_row<true>(a.part_o, a.part_lse, base, n, rows, r, 8 * lane, sk, o, mu, wsum);
    if (8 * lane >= kRopeStart) {
        const float* cs = a.rope_cs + ((size_t)grp * a.s_q + r / a.h_q) * 64;
        const int i0 = (8 * lane - kRopeStart) >> 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float c = cs[i0 + j], sn = cs[32 + i0 + j];
            const float u = o[j >> 1][2 * (j & 1)], w = o[j >> 1][2 * (j & 1) + 1];
            o[j >> 1][2 * (j & 1)] = u * c + w * sn;
            o[j >> 1][2 * (j & 1) + 1] = w * c - u * sn;
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(o[h][e]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float fscale = fmaxf(amax, 1.17549435e-38f) / kE4m3Max;
    const float finv = 1.f / fscale;
    unsigned char* orow = static_cast<unsigned char*>(a.out) + ((size_t)grp * rows + r) * kDv;
    int wv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = fminf(fmaxf(o[h][e] * finv, -kE4m3Max), kE4m3Max);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        wv[h] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
    }
    *reinterpret_cast<uint2*>(orow + 8 * lane) = make_uint2((unsigned)wv[0], (unsigned)wv[1]);
    if (lane == 0) {
        a.out_scale[(size_t)grp * rows + r] = fscale;
        a.lse[(size_t)grp * rows + r] = (mu == -INFINITY) ? -INFINITY : mu + logf(wsum);
    }
}

hipError_t launch_combine_fused(const AttnArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(mla_combine_fused_kernel, dim3(a.batch, (a.M + 3) / 4), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine(const float* part_o, const float* part_lse, const int32_t* prefix,
                          int uniform_splits, int groups, int rows, void* out, float* lse,
                          hipStream_t stream, const float* sinks, int h_q, bool bf16_parts) {
    if (bf16_parts)
        hipLaunchKernelGGL(mla_combine_kernel<true>, dim3(groups, (rows + 3) / 4), dim3(256), 0, stream,
                           part_o, part_lse, prefix, uniform_splits, rows, static_cast<__bf16*>(out), lse,
                           sinks, h_q);
    else
        hipLaunchKernelGGL(mla_combine_kernel<false>, dim3(groups, (rows + 1) / 2), dim3(256), 0, stream,
                           part_o, part_lse, prefix, uniform_splits, rows, static_cast<__bf16*>(out), lse,
                           sinks, h_q);
    return hipGetLastError();
}

}  // namespace mla
