// gfx950 decode kernel for an fp8 paged cache and one 16-row tile (s_q * h_q <= 16), the
// memory-bound shape over 64-token pages of 640-byte records (e4m3 codes of the 576 dims and the
// token's fp32 scale: the fp8 KV cache layout of the decode path, "deepseek-ai/FlashMLA" project
// summary, sections 사용 방법 step 3 and 기술적 세부 사항).
//
// Four independent token streams per workgroup (one per wave, one wave per SIMD) double-buffer
// 32-token chunks (half a page, 20 KB of records) that go HBM -> LDS by direct copies.  Per chunk
// a wave computes S^T = K Q^T for two 16-token tiles (tokens on the MFMA M side, "FlashMLA-ETAP:
// Efficient Transpose Attention Pipeline ...", section 핵심 메커니즘), converting the K fragments
// exactly from e4m3 to bf16 as they are read; the two S^T tiles hold, lane by lane, the P^T B
// operand of one 16x16x32 MFMA per 16 value dims, whose V^T operand comes from a transposing
// 8-bit LDS read in the matching token order.  The token scale multiplies the score and the
// probability before P.V.  Online softmax with a lagging reference, as in the bf16 kernel; the
// four streams merge at the end.
#include "mla_device.h"

namespace mla {

namespace m16f8 {

constexpr int kChunk8 = 32;                    // tokens per chunk: half a page
constexpr int kBuf = kChunk8 * kRec;           // 20 KB of records
constexpr int kOps = kBuf / 1024;              // 20 copies of 64 lanes x 16 B per chunk
constexpr int kStreams = 4;
// LDS read prefetch distances (MFMA steps) of the K and V^T fragments
constexpr int kPfK = 6;
constexpr int kPfV = 6;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_m16_fp8_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[kStreams * 2 * kBuf];   // 160 KB
    const int lane = threadIdx.x & 63;
    const int ts = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);       // stream = wave
    const int g4 = lane >> 4, l16 = lane & 15;
    char* bufs = smem + ts * 2 * kBuf;
    const int item = blockIdx.x;

    // K fragment (A operand of S^T), tile t, step ks: dims 32*ks + 8*g4 of token 16t + l16 =
    // granule 2*ks + g4/2, half g4&1 (kaddr[t][ks&3] + 128*(ks/4): the XOR only touches the low
    // three granule bits)
    int kaddr[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int kr = 16 * t + l16;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) kaddr[t][r4] = kr * kRec + (((2 * r4 + (g4 >> 1)) ^ swz8(kr)) << 4) + (g4 & 1) * 8;
    }
    // V^T fragment (A operand of O^T), dims 16*dt + l16: the transposing read gives this lane 8
    // tokens of granule dt; B operand element j of lane (l16, g4) is token (j < 4 ? 4*g4 + j :
    // 16 + 4*g4 + j - 4), so lane l16 reads rows 4*g4 + l16/2 (l16 < 8) or 16 + 4*g4 + l16/2 - 4
    int vaddr[8];
    {
        const int j = l16 >> 1;
        const int vr = (j < 4) ? 4 * g4 + j : 16 + 4 * g4 + (j - 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) vaddr[e] = vr * kRec + ((e ^ swz8(vr)) << 4) + (l16 & 1) * 8;
    }
    // copies: op j, lane: LDS byte 1024*j + 16*lane = record row rr, slot s, filled from granule
    // s ^ swz8(rr) of the row; c_off is that source offset in a whole chunk
    auto copy_row = [&](int j) { return (64 * j + lane) / 40; };
    auto copy_gran = [&](int j) { const int gg = 64 * j + lane; return ((gg % 40) ^ swz8(gg / 40)) << 4; };
    unsigned c_off[kOps];
#pragma unroll
    for (int j = 0; j < kOps; ++j) c_off[j] = (unsigned)(copy_row(j) * kRec + copy_gran(j));

    bf16x8 qf[18];
    f4 acc[32];
    float m_run, l_run;

    // Q of a segment: the workgroup copies its 16 rows (18 KB, rows past M repeat row 0) into
    // wave 0's second buffer, each wave a quarter; every wave then reads its fragments from there
    char* const qs = smem + kBuf;
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
        const int nch = ceil_div(t1 - t0, kChunk8);

        // Wave ts handles chunks c = ts + 4k: half c & 1 of page (c >> 1) of the segment.  The
        // page numbers come 64 at a time into one register of the wave (lane i: page base + i),
        // the first window from the caller.  A later window's load is waited for inside the
        // reload branch (the empty asm reads it), so the common path carries no pending load: a
        // wait there would be on the whole vector-memory counter, in-flight KV copies included.
        const int lo_page = t0 >> 6;
        int bt_base = 0, win = win0;
        auto page_of = [&](int p) {
            if (p - bt_base >= 64 || p < bt_base) {
                bt_base = p;
                const int np = ceil_div(t1, kPage) - lo_page;
                win = (lane < np - p) ? a.block_table[(size_t)grp * a.max_blocks + lo_page + p + lane] : 0;
                asm volatile("" ::"v"(win));
            }
            return __builtin_amdgcn_readlane(win, p - bt_base);
        };
        // copy chunk c = ts + 4k (32 records, contiguous in HBM) into buffer b; rows past the
        // end repeat the last row (weight 0, finite)
        auto issue = [&](int k, int b) {
            const int c = ts + 4 * k;
            const int tb = t0 + c * kChunk8;
            const int nrows = min(kChunk8, t1 - tb);
            const int page = page_of(c >> 1);
            const char* base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * kRec;
            char* dst = bufs + b * kBuf;
            if (nrows == kChunk8) {
#pragma unroll
                for (int j = 0; j < kOps; ++j) dma16_s(base, c_off[j], dst + 1024 * j);
            } else {
#pragma unroll
                for (int j = 0; j < kOps; ++j) {
                    const int rr = min(copy_row(j), nrows - 1);
                    dma16_s(base, (unsigned)(rr * kRec + copy_gran(j)), dst + 1024 * j);
                }
            }
        };

        if (ts < nch) issue(0, 0);
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
        for (int c = ts; c < nch; c += kStreams, ++k) {
            const char* buf = bufs + (k & 1) * kBuf;
            if (c + kStreams < nch) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of the other buffer done
                issue(k + 1, (k + 1) & 1);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOps) : "memory");   // chunk c landed, c+4 in flight
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            const int tb = t0 + c * kChunk8;
            // S^T of the two tiles over 576 dims: four independent chains.  Step i = 2*ks + t; the
            // K fragment of step i + kPfK is read while step i converts and multiplies, and the
            // schedule interleaves (read, 4 conversions, MFMA) per step so that one wave per SIMD
            // keeps LDS reads in flight behind its MFMAs.
            f4 s2[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t) s2[t][0] = s2[t][1] = f4{0.f, 0.f, 0.f, 0.f};
            auto kread = [&](int i) {
                const int ks = i >> 1, t = i & 1;
                return *reinterpret_cast<const uint2*>(buf + kaddr[t][ks & 3] + 128 * (ks >> 2));
            };
            uint2 kw[36];
#pragma unroll
            for (int i = 0; i < kPfK; ++i) kw[i] = kread(i);
#pragma unroll
            for (int i = 0; i < 36; ++i) {
                if (i + kPfK < 36) kw[i + kPfK] = kread(i + kPfK);
                const int ks = i >> 1, t = i & 1;
                s2[t][ks & 1] = mfma16(fp8x8_to_bf16(kw[i].x, kw[i].y), qf[ks], s2[t][ks & 1]);
                if (i + kPfK < 36) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            // the first V^T fragments, read before the softmax needs the scores
            typedef int v2i __attribute__((ext_vector_type(2)));
            auto vread = [&](int dt) {
                return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i*)(buf + vaddr[dt & 7] + 128 * (dt >> 3)));
            };
            v2i vw[32];
#pragma unroll
            for (int dt = 0; dt < kPfV; ++dt) vw[dt] = vread(dt);
            // mask and scale: token scale * softmax scale (log2 units)
            float x[2][4], tsc[2][4];
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f4 sv = s2[t][0] + s2[t][1];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * t + 4 * g4 + i;
                    const float sc = *reinterpret_cast<const float*>(buf + tok * kRec + ((36 ^ swz8(tok)) << 4));
                    const int tt = tb + tok;
                    const bool valid = (tt < t1) & (tt <= limit);
                    tsc[t][i] = valid ? sc : 0.f;
                    x[t][i] = valid ? sv[i] * (a.scale_log2 * sc) : -INFINITY;
                    mx = fmaxf(mx, x[t][i]);
                }
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
            unsigned pk[4];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = exp2_fast(x[t][i] - m_use);
                    l_run += p[i];
                    p[i] *= tsc[t][i];
                }
                pk[2 * t] = pack_bf16x2(p[0], p[1]);
                pk[2 * t + 1] = pack_bf16x2(p[2], p[3]);
            }
            const bf16x8 pT = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) {
                if (dt + kPfV < 32) vw[dt + kPfV] = vread(dt + kPfV);
                acc[dt] = mfma16(fp8x8_to_bf16((unsigned)vw[dt][0], (unsigned)vw[dt][1]), pT, acc[dt]);
                if (dt + kPfV < 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);
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
        // copy: the first 64 entries of its block-table row from page lo (in bounds of the row;
        // entries past the sequence are never used), its length and split count, and the copy of
        // Q.  All of them are waited for (the empty asm reads the window) before the KV copies
        // start, so no load the compiler tracks is pending behind a copy.
        // (The copy of Q goes first: the compiler's waits on the later loads then cover it.)
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

}  // namespace m16f8

hipError_t launch_decode_m16_fp8(const AttnArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(m16f8::mla_decode_m16_fp8_kernel, dim3(a.num_parts), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
