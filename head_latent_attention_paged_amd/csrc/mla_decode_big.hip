// gfx950 decode kernel for many query rows per KV stream (paged s_q*h_q > 16, sparse h_q > 16).
//
// Each wave owns 32 query rows (two 16-row MFMA tiles), so every K or V^T fragment read
// from LDS feeds two 16x16x32 bf16 MFMAs; the waves of a workgroup cover its rows and share
// one stream of 32-token KV chunks.  Chunks travel HBM -> LDS by direct copies into a ring of
// DEPTH buffers.  The math per chunk is the same as in the other decode kernels: S^T = K Q^T
// with tokens on the MFMA M side ("FlashMLA-ETAP: Efficient Transpose Attention Pipeline ...",
// section 핵심 메커니즘, transposed form), online softmax, O^T += V^T P^T with P^T taken
// straight from the S^T accumulators.
//
// With two wave pairs per workgroup (64 rows) the chunk loop is software-pipelined so that one
// wave per SIMD keeps its MFMA pipe busy: iteration k multiplies S^T(k) while it turns S^T(k-1)
// into probabilities and issues the copies of a later chunk, then (after one barrier) multiplies
// O^T += V^T(k-1) P^T(k-1) while it masks S^T(k) and takes its row maxima.
//
// Sparse fp8: a chunk is 32 gathered records ("deepseek-ai/FlashMLA" project summary,
// section 기술적 세부 사항: fp8 values plus a per-token scale, -1 = unused index).  The raw
// e4m3 codes stay in LDS (half the bytes of bf16) and are converted exactly to bf16 as the
// fragments are read: K with ds_read_b64, V^T with the 8-bit transposing read.  The token
// scale multiplies the token's score and its probability before P.V.
#include "mla_device.h"

#include <type_traits>

namespace mla {

// fp8 record rows in LDS: 40 slots of 16 B (granules 0..35 hold codes, 36 the scale, 37..39
// padding), slot s holding granule s ^ swz8(r), an XOR on the low granule bits that also
// separates rows r and r+16.  The rows of a chunk are contiguous, so one 64-lane copy fills
// 1 KB of it (parts of two rows) and a chunk takes 20 copies with every lane active.
constexpr int kRec8Row = 640;
#ifndef MLA_BIG_SCHED
#define MLA_BIG_SCHED 1
#endif
#ifndef MLA_BIG_PF
#define MLA_BIG_PF 4
#endif
constexpr int kPF = MLA_BIG_PF;   // LDS fragment prefetch distance (MFMA steps)
// The softmax reference of a row is the first finite chunk maximum it sees and never moves
// inside a pass, so the accumulators are touched only by MFMAs.  p = 2^(s - m) <= 2^kRefSlack
// keeps bf16 P and the fp32 sums finite; a row whose scores outgrow the reference by more
// (scores spanning over 44 nats) makes the workgroup finish the pass and run it again with each
// row's maximum over the whole segment as reference: at most two passes.
constexpr float kRefSlack = 64.f;
// LDS layouts, chosen by measuring the kernels' read patterns on gfx950 (64 banks): bf16 region A
// holds dims 0..511 of a row in 1 KB at a 1056-byte row stride, unswizzled, which keeps both the
// 16 rows x 64 B of a K read (ds_read_b128) and the 8 rows x 32 B of a V^T transposing read
// conflict-free.  Region B (the RoPE dims, 128 B rows): slot = granule ^ swzB(r).  fp8 rows
// (640 B): slot = granule ^ swz8(r) keeps the 16 rows of a K read and of a V^T tr8 read apart.
constexpr int kRowA16 = 1056;
constexpr int kRegionB16 = kChunk * kRowA16;
constexpr int kChunk16 = kRegionB16 + kChunk * 128;
__device__ __forceinline__ int swzB(int r) { return (r >> 1) & 7; }

// An all-zero record: unused index entries are copied from it, so a chunk always costs the same
// copies (exact s_waitcnt accounting) and its zero-weight V rows are finite.
__device__ __attribute__((aligned(16))) const unsigned char kZeroRecord[kRec8Row] = {0};

// Workgroup: PAIRS pairs of waves sharing one stream of chunks.  A pair owns 32 query rows;
// in each 32-token chunk wave h (0/1) of the pair computes S^T for tokens 16h..16h+15 and
// O^T for value dims 256h..256h+255, so it holds 32 rows of Q (B operand) and half the O^T
// accumulators.  The pair exchanges row maxima and its halves of P^T through LDS.
template <bool SPARSE, int PAIRS>
struct BigCfg {
    static constexpr int WAVES = 2 * PAIRS;
    static constexpr int ROWS_WG = 32 * PAIRS;
    static constexpr bool PIPELINED = PAIRS == 2;
    static constexpr int BUF = SPARSE ? kChunk * kRec8Row : kChunk16;
    // ring slots.  Pipelined: chunk k-1 (P.V), k (Q.K^T) and DEPTH-2 chunks in flight.  Serial
    // (one pair, leaving room for a second workgroup per CU): DEPTH-1 chunks in flight.
    static constexpr int DEPTH = PAIRS == 2 ? (SPARSE ? 6 : 4) : (SPARSE ? 3 : 2);
    static constexpr int RING = DEPTH * BUF;
    // copies per wave per chunk: bf16 32 rows of region A + 4 KB of region B; fp8 20 KB
    static constexpr int OPS = (SPARSE ? kChunk * kRec8Row / 1024 : kChunk + 4) / WAVES;
    static constexpr int MAIN = RING;
    static constexpr int XCH = WAVES * 2 * 16 * 4;                     // row maxima / sums [wave][n][row]
    static constexpr int PEX = WAVES * 2 * 64 * 8;                     // P^T halves [wave][n][lane]
    static constexpr int IDX = SPARSE ? kMaxSparseSplit * 4 : 0;       // a split's index list
    static constexpr int PAGES = SPARSE ? 0 : WAVES * 64 * 4;            // per-wave page windows
    static constexpr int FLAGS = 64;                                     // per-wave restart votes
    static constexpr int SINK = WAVES * 64 * 4;                         // targets of masked-off lanes
    static constexpr int LDS = MAIN + XCH + PEX + IDX + PAGES + FLAGS + SINK;
};

template <bool SPARSE, int PAIRS, bool SHARED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_big_kernel(const AttnArgs a) {
    using C = BigCfg<SPARSE, PAIRS>;
    constexpr int DEPTH = C::DEPTH;
    constexpr int WAVES = C::WAVES;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    float* xch = reinterpret_cast<float*>(smem + C::MAIN);
    uint2* pex = reinterpret_cast<uint2*>(smem + C::MAIN + C::XCH);
    int* lidx = reinterpret_cast<int*>(smem + C::MAIN + C::XCH + C::PEX);
    int* lpages = reinterpret_cast<int*>(smem + C::MAIN + C::XCH + C::PEX + C::IDX);
    int* votes = reinterpret_cast<int*>(smem + C::MAIN + C::XCH + C::PEX + C::IDX + C::PAGES);
    float* sink = reinterpret_cast<float*>(smem + C::MAIN + C::XCH + C::PEX + C::IDX + C::PAGES + C::FLAGS);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = wave & 1;                      // token half (QK) and dim half (PV)
    const int pair = wave >> 1;
    const int partner = wave ^ 1;
    const int g4 = lane >> 4, l16 = lane & 15;
    char* ring = smem;
    // lanes that must not store write their own word of the sink instead (no branch)
    float* my_sink = sink + wave * 64 + lane;

    // ---- work item -> (part or sparse split, row group); row groups of one item share an XCD
    const int R = ceil_div(a.M, C::ROWS_WG);
    const int n_items = SPARSE ? a.batch * a.num_parts : a.num_parts;
    int item, rg;
    xcd_item(blockIdx.x, n_items, R, item, rg);
    const int rbase = rg * C::ROWS_WG + pair * 32;
    // row groups that re-read the same KV keep it in L2 (default policy); a single reader
    // streams it (nontemporal)
    auto copy = [&](const void* g, const void* l) {
        if constexpr (SHARED) dma16_shared(g, l);
        else dma16(g, l);
    };

    // fragment addresses that do not depend on the chunk
    const int krow = 16 * h + l16;               // this wave's K rows: tokens 16h..16h+15
    int kaddr = 0, kaddrB[2];                    // bf16: region A + 64*ks, region B [ks&1]
    int vaddr[2];                                // bf16 tr16: [half] + 32*dt
    // fp8: the XOR of the row layout only touches the low 3 granule bits, so fragment offsets
    // repeat with a constant 128 B stride: K step ks uses k8addr[ks&3] + 128*(ks/4), V^T tile
    // dt uses v8addr[dt&7] + 128*(dt/8)
    int k8addr[4], v8addr[8];
    if constexpr (!SPARSE) {
        // K step ks reads dims 32*ks + 8*g4 .. +7 of row krow (ks >= 16: the RoPE dims)
        kaddr = krow * kRowA16 + g4 * 16;
#pragma unroll
        for (int par = 0; par < 2; ++par)
            kaddrB[par] = kRegionB16 + krow * 128 + (((4 * par + g4) ^ swzB(krow)) << 4);
        // V^T tile dt: lane supplies row 4*g4 + l16/4 (+16 for the upper tokens), dims
        // 16*dt + 8*((l16&3)>>1) + 4*(l16&1)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            vaddr[hf] = (4 * g4 + (l16 >> 2) + 16 * hf) * kRowA16 + ((l16 & 3) >> 1) * 16 + (l16 & 1) * 8;
    } else {
        // K: lane (g4, l16) reads 8 codes of token krow at dims 16*ks + 8*g4 .. (granule
        // 2*ks + g4/2, half g4&1)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            k8addr[r] = krow * kRec8Row + (((2 * r + (g4 >> 1)) ^ swz8(krow)) << 4) + (g4 & 1) * 8;
        // tr8: source lane s of group g supplies token (s/2 < 4 ? 4g + s/2 : 16 + 4g + s/2 - 4)
        const int j = l16 >> 1;
        const int v8row = (j < 4) ? 4 * g4 + j : 16 + 4 * g4 + (j - 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) v8addr[e] = v8row * kRec8Row + ((e ^ swz8(v8row)) << 4) + (l16 & 1) * 8;
    }

    bf16x8 qf[2][18];
    f4 acc[16][2];
    float m_run[2], l_run[2];
    float m_lane[2];   // largest score this lane has seen in the pass (a restart's reference)

    auto run_segment = [&](int grp, int t0, int t1, int L, bool final_out, int slot) {
        const int nch = ceil_div(t1 - t0, kChunk);
        // ---- Q fragments (B operand of S^T): row l16 of tile n, dims 8*g4 + 32*ks
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int r = rbase + 16 * n + l16;
            const char* qrow = static_cast<const char*>(a.q) + ((size_t)grp * a.M + (r < a.M ? r : 0)) * (kDqk * 2);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                uint4 v = *reinterpret_cast<const uint4*>(qrow + (ks * 32 + g4 * 8) * 2);
                if (r >= a.M) v = make_uint4(0, 0, 0, 0);
                qf[n][ks] = __builtin_bit_cast(bf16x8, v);
            }
            m_run[n] = -INFINITY;
        }
        int limit[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) limit[n] = a.causal ? (L - a.s_q + (rbase + 16 * n + l16) / a.h_q) : (L - 1);

        // sparse: the split's index list goes to LDS once (no vector loads inside the pipeline)
        if constexpr (SPARSE) {
            for (int e = threadIdx.x; e < t1 - t0; e += C::WAVES * 64) lidx[e] = a.indices[(size_t)grp * a.topk + t0 + e];
            __syncthreads();
        }

        // paged: page numbers of the segment, 64 at a time into a per-wave LDS window (a lookup
        // then never waits on the vector-memory counter, which also counts the KV copies)
        int bt_base = -1000000;
        auto page_of = [&](int p) {
            int* win = lpages + wave * 64;
            if (p - bt_base >= 64 || p < bt_base) {
                bt_base = p;
                const int np = ceil_div(t1, kPage) - (t0 >> 6);
                const int v = (lane < np - p) ? a.block_table[(size_t)grp * a.max_blocks + (t0 >> 6) + p + lane] : 0;
                win[lane] = v;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            return __builtin_amdgcn_readfirstlane(win[p - bt_base]);
        };

        // ---- copies of one chunk: each wave copies every WAVES-th row.  A plan holds what
        // does not depend on the copy (so the copies can be spread over the MFMAs); chunks past
        // the segment's end re-copy its last chunk into their (unused) slot, which keeps the
        // number of copies per chunk fixed.
        struct Plan {
            const char* base;                      // paged: first row of the chunk in HBM
            int idx[SPARSE ? C::OPS : 1];          // sparse: record of the row this lane fills, per copy
            char* dst;
            int nrows;
        };
        auto plan_for = [&](int c) {
            Plan p;
            const int cc = min(c, nch - 1);
            p.dst = ring + (c % DEPTH) * C::BUF;
            const int tb = t0 + cc * kChunk;
            p.nrows = min(kChunk, t1 - tb);
            if constexpr (!SPARSE) {
                const int page = page_of(cc >> 1);
                p.base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * kRowBytes;
            } else {
                p.base = nullptr;
                // recomputed per chunk on purpose: hoisted, these addresses would not fit in registers
                int ln = lane;
                asm volatile("" : "+v"(ln));
#pragma unroll
                for (int j = 0; j < C::OPS; ++j) {
                    const int row = (64 * (wave + WAVES * j) + ln) / 40;   // row of the granule this lane fills
                    const int v = lidx[cc * kChunk + row];     // inside the list; stale past its end
                    p.idx[j] = row < p.nrows ? v : -1;
                }
            }
            return p;
        };
        auto copy_op = [&](const Plan& p, int j) {
            if constexpr (!SPARSE) {
                const int q = wave + WAVES * j;
                if (j < kChunk / WAVES) {   // region A rows (WAVES divides kChunk)
                    const int rr = min(q, p.nrows - 1);
                    copy(p.base + rr * kRowBytes + (lane << 4), p.dst + q * kRowA16);
                } else {
                    const int sl = (q - kChunk) * 64 + lane;
                    const int row = sl >> 3;
                    const int rr = min(row, p.nrows - 1);
                    copy(p.base + rr * kRowBytes + (64 + ((sl & 7) ^ swzB(row))) * 16,
                         p.dst + kRegionB16 + (q - kChunk) * 1024);
                }
            } else {
                const int gg = 64 * (wave + WAVES * j) + lane;
                const int row = gg / 40, slot_g = gg - 40 * row;
                const char* rec = p.idx[j] >= 0 ? static_cast<const char*>(a.kv) + (size_t)p.idx[j] * kRec
                                                : reinterpret_cast<const char*>(kZeroRecord);
                copy(rec + ((slot_g ^ swz8(row)) << 4), p.dst + 1024 * (wave + WAVES * j));
            }
        };

        // ---- LDS fragments
        auto kfrag = [&](const char* buf, int ks) -> bf16x8 {
            if constexpr (!SPARSE) {
                const int off = ks < 16 ? kaddr + 64 * ks : kaddrB[ks & 1];
                return *reinterpret_cast<const bf16x8*>(buf + off);
            } else {
                const uint2 w = *reinterpret_cast<const uint2*>(buf + k8addr[ks & 3] + 128 * (ks >> 2));
                return fp8x8_to_bf16(w.x, w.y);
            }
        };
        auto vfrag = [&](const char* buf, int dt) -> bf16x8 {    // dt: global 16-dim tile 0..31
            if constexpr (!SPARSE) {
                const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr[0] + 32 * dt));
                const short4v v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr[1] + 32 * dt));
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
                typedef int v2i __attribute__((ext_vector_type(2)));
                const v2i w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i*)(buf + v8addr[dt & 7] + 128 * (dt >> 3)));
                return fp8x8_to_bf16((unsigned)w[0], (unsigned)w[1]);
            }
        };

        // S^T partial products of chunk c for this wave's 16 tokens: [n][ks&1], four independent
        // MFMA chains.  side(ks) runs between the steps (work of other stages); fragments are
        // read kPF steps ahead of their MFMAs, since one wave per SIMD leaves nothing else to
        // hide the LDS latency.
        auto qk = [&](int c, f4 (&s2)[2][2], auto&& side) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
#pragma unroll
            for (int n = 0; n < 2; ++n) s2[n][0] = s2[n][1] = f4{0.f, 0.f, 0.f, 0.f};
            bf16x8 kf[kPF];
#pragma unroll
            for (int i = 0; i < kPF - 1; ++i) kf[i] = kfrag(buf, i);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                if (ks + kPF - 1 < 18) kf[(ks + kPF - 1) % kPF] = kfrag(buf, ks + kPF - 1);
#pragma unroll
                for (int n = 0; n < 2; ++n) s2[n][ks & 1] = mfma16(kf[ks % kPF], qf[n][ks], s2[n][ks & 1]);
                side(ks);
                if (MLA_BIG_SCHED) __builtin_amdgcn_sched_barrier(0);
            }
        };
        // O^T[256h + ..][row] += V^T P^T over chunk c's 32 tokens; side(dt) between the steps
        auto pv = [&](int c, const bf16x8 (&pT)[2], auto&& side) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            bf16x8 vf[kPF];
#pragma unroll
            for (int i = 0; i < kPF - 1; ++i) vf[i] = vfrag(buf, 16 * h + i);
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) {
                if (dt + kPF - 1 < 16) vf[(dt + kPF - 1) % kPF] = vfrag(buf, 16 * h + dt + kPF - 1);
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[dt][n] = mfma16(vf[dt % kPF], pT[n], acc[dt][n]);
                side(dt);
                if (MLA_BIG_SCHED) __builtin_amdgcn_sched_barrier(0);
            }
        };

        // ---- softmax stages of one chunk, in steps that can be spread over MFMAs
        struct Scores {
            f4 s[2];        // masked, scaled (log2 units) S^T values of this wave's 16 tokens
            float mx[2];    // row maxima (only taken when a row has no reference yet, or at a restart)
            float tsc[4];   // sparse: token scales
            bool ok[4];     // token inside the segment and a real index
            bool outgrown;  // a score of a row with a reference exceeds it by more than kRefSlack
            bool need_max;  // (wave-uniform) some row has no reference yet
        };
        // Row maxima are only needed while a row has no reference (its first chunk) and at a
        // restart; otherwise each lane just compares its own scores with the reference.
        // step 0: sum the chains; 1: token validity and scales; 2/3: mask and scale tile n and
        // test it against the reference
        auto mask_step = [&](int step, int c, const f4 (&s2)[2][2], Scores& S) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            const int tb = t0 + c * kChunk;
            if (step == 0) {
#pragma unroll
                for (int n = 0; n < 2; ++n) S.s[n] = s2[n][0] + s2[n][1];
                S.need_max = __builtin_amdgcn_ballot_w64(m_run[0] == -INFINITY || m_run[1] == -INFINITY) != 0;
                S.outgrown = false;
            } else if (step == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * h + 4 * g4 + i;
                    if constexpr (SPARSE) {
                        const int v = lidx[c * kChunk + tok];   // inside the list; stale past its end
                        const float sc = *reinterpret_cast<const float*>(buf + tok * kRec8Row + ((36 ^ swz8(tok)) << 4));
                        S.ok[i] = tb + tok < t1 && v >= 0;
                        S.tsc[i] = S.ok[i] ? sc : 0.f;
                    } else {
                        S.ok[i] = tb + tok < t1;
                        S.tsc[i] = 1.f;
                    }
                }
            } else if (step == 2 || step == 3) {
                const int n = step - 2;
                const float cap = m_run[n] + kRefSlack;      // -inf while the row has no reference
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bool valid = S.ok[i];
                    if constexpr (!SPARSE) valid = valid && (tb + 16 * h + 4 * g4 + i <= limit[n]);
                    const float f = SPARSE ? a.scale_log2 * S.tsc[i] : a.scale_log2;
                    S.s[n][i] = valid ? S.s[n][i] * f : -INFINITY;
                    S.outgrown = S.outgrown || (m_run[n] != -INFINITY && S.s[n][i] > cap);
                    m_lane[n] = fmaxf(m_lane[n], S.s[n][i]);
                }
            }
        };
        // this wave's row maxima of S (cross-lane) into LDS for the partner
        auto max_to_lds = [&](Scores& S) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                S.mx[n] = fmaxf(fmaxf(S.s[n][0], S.s[n][1]), fmaxf(S.s[n][2], S.s[n][3]));
                S.mx[n] = fmaxf(S.mx[n], __shfl_xor(S.mx[n], 16));
                S.mx[n] = fmaxf(S.mx[n], __shfl_xor(S.mx[n], 32));
                *(g4 == 0 ? &xch[(wave * 2 + n) * 16 + l16] : my_sink) = S.mx[n];
            }
        };
        // after a barrier: the pair's row maxima
        auto pair_max = [&](Scores& S) {
#pragma unroll
            for (int n = 0; n < 2; ++n) S.mx[n] = fmaxf(S.mx[n], xch[(partner * 2 + n) * 16 + l16]);
        };
        // After a barrier: step 0 gives rows without a reference the pair's maximum; 1 votes;
        // 2/3 probabilities of tile n; 4 stores this wave's P^T half; 5 stores the vote.
        struct Probs {
            uint2 mine[2];
            bool vote;
        };
        auto prob_step = [&](int step, Scores& S, Probs& P) {
            if (step == 0) {
                if (S.need_max) {
                    pair_max(S);
#pragma unroll
                    for (int n = 0; n < 2; ++n)
                        if (m_run[n] == -INFINITY) m_run[n] = S.mx[n];     // acc and l are still exactly 0
                }
            } else if (step == 1) {
                P.vote = __builtin_amdgcn_ballot_w64(S.outgrown) != 0;
            } else if (step == 2 || step == 3) {
                const int n = step - 2;
                const float m_use = (m_run[n] == -INFINITY) ? 0.f : m_run[n];
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = exp2_fast(S.s[n][i] - m_use);
                    l_run[n] += p[i];
                    if constexpr (SPARSE) p[i] *= S.tsc[i];
                }
                P.mine[n] = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
            } else if (step == 4) {
#pragma unroll
                for (int n = 0; n < 2; ++n) pex[(wave * 2 + n) * 64 + lane] = P.mine[n];
            } else if (step == 5) {
                *(lane == 0 ? reinterpret_cast<float*>(&votes[wave]) : my_sink) = __int_as_float(P.vote ? 1 : 0);
            }
        };
        // after the barrier that follows prob_step: any vote in the workgroup?  Else this wave's
        // B operands of O^T += V^T P^T
        auto any_vote = [&]() {
            int any = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) any |= votes[w];
            return __builtin_amdgcn_readfirstlane(any) != 0;
        };
        auto p_operands = [&](const Probs& P, bf16x8 (&pT)[2]) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const uint2 other = pex[(partner * 2 + n) * 64 + lane];
                const uint4 pk = h == 0 ? make_uint4(P.mine[n].x, P.mine[n].y, other.x, other.y)
                                        : make_uint4(other.x, other.y, P.mine[n].x, P.mine[n].y);
                pT[n] = __builtin_bit_cast(bf16x8, pk);
            }
        };
        auto no_side = [](int) {};

        // ---- passes over the segment (a second one only after a restart vote).  A vote does not
        // end the pass early: the pass runs to its end (its results are discarded), so m_lane sees
        // every score of the segment and the second pass, whose reference is that maximum,
        // cannot vote.
        for (int pass = 0;; ++pass) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                m_lane[n] = -INFINITY;
                l_run[n] = 0.f;
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) acc[dt][n] = f4{0.f, 0.f, 0.f, 0.f};
            }
            bool restart = false;
            Scores S;
            if constexpr (C::PIPELINED) {
                // DEPTH-2 chunks ahead.  Every chunk slot gets exactly C::OPS copies per wave, so
                // chunk k has landed once at most DEPTH-3 later chunks' copies are outstanding.
                constexpr int AHEAD = DEPTH - 2;
#pragma unroll
                for (int c = 0; c < AHEAD; ++c) {
                    const Plan p = plan_for(c);
#pragma unroll
                    for (int j = 0; j < C::OPS; ++j) copy_op(p, j);
                }
                auto wait_chunk = [&]() {
                    if constexpr (AHEAD - 1 == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((AHEAD - 1) * C::OPS) : "memory");
                };
                // chunk 0: Q.K^T (copies of chunk AHEAD spread over it), mask and maxima
                wait_chunk();
                __syncthreads();
                {
                    const Plan p = plan_for(AHEAD);
                    f4 s2[2][2];
                    qk(0, s2, [&](int ks) {
                        if ((ks & 1) == 0 && ks / 2 < C::OPS) copy_op(p, ks / 2);
                    });
#pragma unroll
                    for (int step = 0; step < 4; ++step) mask_step(step, 0, s2, S);
                    if (S.need_max) max_to_lds(S);
                }
                for (int k = 1; k < nch; ++k) {
                    wait_chunk();
                    // chunk k in LDS; maxima of chunk k-1 visible; slot (k-2) % DEPTH free
                    __syncthreads();
                    const Plan p = plan_for(k + AHEAD);
                    Probs P;
                    f4 s2[2][2];
                    // S^T(k) on the MFMAs while chunk k-1 becomes probabilities and chunk
                    // k+AHEAD is copied
                    qk(k, s2, [&](int ks) {
                        if ((ks & 1) == 0 && ks / 2 < C::OPS) copy_op(p, ks / 2);
                        if (ks == 1) prob_step(0, S, P);
                        if (ks == 3) prob_step(1, S, P);
                        if (ks == 5) prob_step(2, S, P);
                        if (ks == 7) prob_step(3, S, P);
                        if (ks == 9) prob_step(4, S, P);
                        if (ks == 10) prob_step(5, S, P);
                    });
                    __syncthreads();               // P^T halves and votes of chunk k-1 visible
                    restart = restart || any_vote();
                    bf16x8 pT[2];
                    p_operands(P, pT);
                    // O^T += V^T P^T (k-1) on the MFMAs while S^T(k) is masked
                    pv(k - 1, pT, [&](int dt) {
                        if (dt < 4) mask_step(dt, k, s2, S);
                    });
                    if (S.need_max) max_to_lds(S);
                }
                {
                    __syncthreads();               // maxima of the last chunk visible
                    Probs P;
#pragma unroll
                    for (int step = 0; step < 6; ++step) prob_step(step, S, P);
                    __syncthreads();
                    restart = restart || any_vote();
                    if (!restart) {
                        bf16x8 pT[2];
                        p_operands(P, pT);
                        pv(nch - 1, pT, no_side);
                    }
                }
            } else {
                // one pair: DEPTH-1 chunks in flight, the stages of a chunk back to back
#pragma unroll
                for (int c = 0; c < DEPTH - 1; ++c) {
                    const Plan p = plan_for(c);
#pragma unroll
                    for (int j = 0; j < C::OPS; ++j) copy_op(p, j);
                }
                for (int k = 0; k < nch; ++k) {
                    if constexpr (DEPTH - 2 == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DEPTH - 2) * C::OPS) : "memory");
                    __syncthreads();               // chunk k is in LDS; slot k-1 is no longer read
                    {
                        const Plan p = plan_for(k + DEPTH - 1);
#pragma unroll
                        for (int j = 0; j < C::OPS; ++j) copy_op(p, j);
                    }
                    f4 s2[2][2];
                    qk(k, s2, no_side);
#pragma unroll
                    for (int step = 0; step < 4; ++step) mask_step(step, k, s2, S);
                    if (S.need_max) max_to_lds(S);
                    __syncthreads();
                    Probs P;
#pragma unroll
                    for (int step = 0; step < 6; ++step) prob_step(step, S, P);
                    __syncthreads();
                    restart = restart || any_vote();
                    bf16x8 pT[2];
                    p_operands(P, pT);
                    pv(k, pT, no_side);
                }
            }
            // the copies past the segment's end (or those in flight at a restart) land first
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // (the second pass cannot vote; the bound on the passes is a guard)
            if (!restart || pass == 1) break;
            // start over with each row's maximum over the whole pass as reference
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                S.mx[n] = fmaxf(m_lane[n], __shfl_xor(m_lane[n], 16));
                S.mx[n] = fmaxf(S.mx[n], __shfl_xor(S.mx[n], 32));
                *(g4 == 0 ? &xch[(wave * 2 + n) * 16 + l16] : my_sink) = S.mx[n];
            }
            __syncthreads();
            pair_max(S);
#pragma unroll
            for (int n = 0; n < 2; ++n) m_run[n] = fmaxf(m_run[n], S.mx[n]);
            __syncthreads();
        }

        // ---- row sums of the pair (both halves share the reference m), then the output
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            l_run[n] += __shfl_xor(l_run[n], 16);
            l_run[n] += __shfl_xor(l_run[n], 32);
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < 2; ++n)
            if (g4 == 0) xch[(wave * 2 + n) * 16 + l16] = l_run[n];
        __syncthreads();
#pragma unroll
        for (int n = 0; n < 2; ++n) l_run[n] += xch[(partner * 2 + n) * 16 + l16];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int r = rbase + 16 * n + l16;
            const float l = l_run[n];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const float lse_v = l > 0.f ? (m_run[n] + __log2f(l)) * kLn2 : -INFINITY;
            if (r < a.M) {
                if (final_out) {
                    __bf16* orow = static_cast<__bf16*>(a.out) + ((size_t)grp * a.M + r) * kDv + 256 * h + 4 * g4;
#pragma unroll
                    for (int dt = 0; dt < 16; ++dt) {
                        const f4 v = acc[dt][n] * inv;
                        *reinterpret_cast<uint2*>(orow + dt * 16) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
                    if (g4 == 0 && h == 0) a.lse[(size_t)grp * a.M + r] = lse_v;
                } else {
                    float* prow = a.part_o + ((size_t)slot * a.M + r) * kDv + 256 * h + 4 * g4;
#pragma unroll
                    for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<f4*>(prow + dt * 16) = acc[dt][n] * inv;
                    if (g4 == 0 && h == 0) a.part_lse[(size_t)slot * a.M + r] = lse_v;
                }
            }
        }
        __syncthreads();                    // LDS (ring, index list, exchanges) free for the next segment
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
        }
    } else {
        const int grp = item / a.num_parts;
        const int split = item % a.num_parts;
        const int e0 = split * a.split_len;
        const int e1 = min(e0 + a.split_len, a.topk);
        if (e0 < e1) run_segment(grp, e0, e1, 0, a.num_parts == 1, grp * a.num_parts + split);
    }
}

template <bool SPARSE, int PAIRS>
static hipError_t launch_big_t(const AttnArgs& a, int items, hipStream_t stream) {
    using C = BigCfg<SPARSE, PAIRS>;
    const int R = (a.M + C::ROWS_WG - 1) / C::ROWS_WG;
    if (R > 1)
        hipLaunchKernelGGL((mla_decode_big_kernel<SPARSE, PAIRS, true>), dim3(items * R), dim3(C::WAVES * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((mla_decode_big_kernel<SPARSE, PAIRS, false>), dim3(items * R), dim3(C::WAVES * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_big(const AttnArgs& a, bool sparse, hipStream_t stream) {
    const int items = sparse ? a.batch * a.num_parts : a.num_parts;
    // sparse calls come here with 16 < h_q <= 32 only (more heads take the row-split kernel)
    if (sparse) return big_pairs(a.M) == 1 ? launch_big_t<true, 1>(a, items, stream) : hipErrorInvalidValue;
    if (big_pairs(a.M) == 1) return launch_big_t<false, 1>(a, items, stream);
    return launch_big_t<false, 2>(a, items, stream);
}

}  // namespace mla
