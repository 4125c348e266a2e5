// gfx950 decode kernel for many query rows per KV stream (paged s_q*h_q > 16, sparse h_q > 16).
//
// Each wave owns 32 query rows (two 16-row MFMA tiles), so every K or V^T fragment read
// from LDS feeds two 16x16x32 bf16 MFMAs; the waves of a workgroup cover its rows and share
// one stream of 32-token KV chunks.  Chunks travel HBM -> LDS by direct nontemporal copies into
// a ring of DEPTH buffers, DEPTH-1 chunks ahead of the one being multiplied, with one
// workgroup barrier per chunk.  The math per chunk is the same as in the other decode
// kernels: S^T = K Q^T with tokens on the MFMA M side ("FlashMLA-ETAP: Efficient Transpose
// Attention Pipeline ...", section 방법론 / 핵심 메커니즘, transposed form), a lagging-
// reference online softmax, O^T += V^T P^T with P^T taken straight from the S^T
// accumulators.
//
// Sparse fp8: a chunk is 32 gathered records ("deepseek-ai/FlashMLA" project summary,
// section 기술적 세부 사항: fp8 values plus a per-token scale, -1 = unused index).  The raw
// e4m3 codes stay in LDS (half the bytes of bf16) and are converted exactly to bf16 as the
// fragments are read: K with ds_read_b64, V^T with the 8-bit transposing read.  The token
// scale multiplies the token's score and its probability before P.V.
#include "mla_device.h"

namespace mla {

// fp8 record rows in LDS: 40 slots of 16 B (granules 0..35 hold codes, 36 the scale) with an
// XOR on the low granule bits that also separates rows r and r+16.
constexpr int kRec8Row = 640;
constexpr int kPF = 4;       // LDS fragment prefetch distance (MFMA steps)
// The softmax reference of a row is the first finite chunk maximum it sees and never moves
// inside a pass, so the accumulators are touched only by MFMAs.  p = 2^(s - m) <= 2^kRefSlack
// keeps bf16 P and the fp32 sums finite; a row whose scores outgrow the reference by more
// (scores spanning over 44 nats) makes the workgroup restart the segment with the larger
// reference.
constexpr float kRefSlack = 64.f;
__device__ __forceinline__ int swz8(int r) { return (((r & 3) << 1) | ((r >> 2) & 1)) ^ ((r >> 4) & 1); }

// An all-zero record: unused index entries and rows past a split's end are copied from it,
// so every row of a chunk costs exactly one copy (exact s_waitcnt accounting) and its
// (zero-weight) V row is finite.
__device__ __attribute__((aligned(16))) const unsigned char kZeroRecord[kRec8Row] = {0};

// 8 e4m3 codes (two dwords) -> 8 bf16, exact
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(unsigned lo, unsigned hi) {
#define MLA_CVT(w, h) __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, h))
    const uint4 v = make_uint4(MLA_CVT(lo, false), MLA_CVT(lo, true), MLA_CVT(hi, false), MLA_CVT(hi, true));
#undef MLA_CVT
    return __builtin_bit_cast(bf16x8, v);
}

// Workgroup: PAIRS pairs of waves sharing one stream of chunks.  A pair owns 32 query rows;
// in each 32-token chunk wave h (0/1) of the pair computes S^T for tokens 16h..16h+15 and
// O^T for value dims 256h..256h+255, so it holds 32 rows of Q (B operand) and half the O^T
// accumulators.  The pair exchanges row maxima and its halves of P^T through LDS.
template <bool SPARSE, int PAIRS>
struct BigCfg {
    static constexpr int WAVES = 2 * PAIRS;
    static constexpr int ROWS_WG = 32 * PAIRS;
    static constexpr int BUF = SPARSE ? kChunk * kRec8Row : kChunkBytes;
    // ring depth: two pairs fill a compute unit alone; one pair leaves room for a second block
    static constexpr int DEPTH = PAIRS == 2 ? (SPARSE ? 6 : 4) : (SPARSE ? 3 : 2);
    static constexpr int RING = DEPTH * BUF;
    static constexpr int OPS = (SPARSE ? kChunk : kChunk + 4) / WAVES;  // copies per wave per chunk
    static constexpr int MAIN = RING;
    static constexpr int XCH = WAVES * 2 * 16 * 4;                     // row maxima / sums [wave][n][row]
    static constexpr int PEX = WAVES * 2 * 64 * 8;                     // P^T halves [wave][n][lane]
    static constexpr int IDX = SPARSE ? kMaxSparseSplit * 4 : 0;       // a split's index list
    static constexpr int PAGES = SPARSE ? 0 : WAVES * 64 * 4;            // per-wave page windows
    static constexpr int FLAGS = 64;                                     // per-wave restart votes
    static constexpr int LDS = MAIN + XCH + PEX + IDX + PAGES + FLAGS;
};

template <bool SPARSE, int PAIRS>
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

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = wave & 1;                      // token half (QK) and dim half (PV)
    const int pair = wave >> 1;
    const int partner = wave ^ 1;
    const int g4 = lane >> 4, l16 = lane & 15;
    char* ring = smem;

    // ---- work item -> (part or sparse split, row group); row groups of one item share an XCD
    const int R = ceil_div(a.M, C::ROWS_WG);
    const int n_items = SPARSE ? a.batch * a.num_parts : a.num_parts;
    int item, rg;
    {
        const int bid = blockIdx.x;
        if ((n_items & 7) == 0) {
            const int xcd = bid & 7, k = bid >> 3;
            item = (k / R) * 8 + xcd;
            rg = k % R;
        } else {
            item = bid / R;
            rg = bid % R;
        }
    }
    const int rbase = rg * C::ROWS_WG + pair * 32;
    const bool kv_shared = R > 1;              // row groups re-read the same KV: keep it in L2

    // fragment addresses that do not depend on the chunk
    const int krow = 16 * h + l16;               // this wave's K rows: tokens 16h..16h+15
    int kaddr[2], kaddrB[2];                     // bf16: [ks&1] (+128 per ks/2 in region A)
    int vaddr[2][4];                             // bf16 tr16: [half][dt&3] (+128 per dt/4)
    int v8row = 0;                               // fp8 tr8: source token row of this lane
    if constexpr (!SPARSE) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            kaddr[par] = lds_a(krow, 4 * par + g4);
            kaddrB[par] = lds_b(krow, 4 * par + g4);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int d4 = 0; d4 < 4; ++d4) {
                const int row = 4 * g4 + (l16 >> 2) + 16 * hf;
                vaddr[hf][d4] = lds_a(row, 2 * d4 + ((l16 & 3) >> 1)) + (l16 & 1) * 8;
            }
    } else {
        // tr8: source lane s of group g supplies token (s/2 < 4 ? 4g + s/2 : 16 + 4g + s/2 - 4)
        const int j = l16 >> 1;
        v8row = (j < 4) ? 4 * g4 + j : 16 + 4 * g4 + (j - 4);
    }

    bf16x8 qf[2][18];
    f4 acc[16][2];
    float m_run[2], l_run[2];

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

        // copy chunk c of the segment into ring slot c % DEPTH; each wave copies every WAVES-th row
        auto issue_with = [&](int c, auto shared) {
            auto copy = [&](const void* g, const void* l) {
                if constexpr (decltype(shared)::value) dma16_shared(g, l);
                else dma16(g, l);
            };
            char* dst = ring + (c % DEPTH) * C::BUF;
            const int tb = t0 + c * kChunk;
            const int nrows = min(kChunk, t1 - tb);
            if constexpr (!SPARSE) {
                const int page = page_of(c >> 1);
                const char* base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * kRowBytes;
#pragma unroll
                for (int j = 0; j < C::OPS; ++j) {
                    const int q = wave + WAVES * j;
                    if (j < kChunk / WAVES) {   // region A rows (WAVES divides kChunk)
                        const int rr = min(q, nrows - 1);
                        copy(base + rr * kRowBytes + ((lane ^ swz(q)) << 4), dst + q * kRowA);
                    } else {
                        const int sl = (q - kChunk) * 64 + lane;
                        const int row = sl >> 3;
                        const int rr = min(row, nrows - 1);
                        copy(base + rr * kRowBytes + (64 + ((sl & 7) ^ swz(row))) * 16,
                             dst + kRegionB + (q - kChunk) * 1024);
                    }
                }
            } else {
                const char* kvb = static_cast<const char*>(a.kv);
#pragma unroll
                for (int j = 0; j < C::OPS; ++j) {
                    const int row = wave + WAVES * j;
                    const int idx = row < nrows ? lidx[c * kChunk + row] : -1;
                    const char* src = idx >= 0 ? kvb + (size_t)idx * kRec : reinterpret_cast<const char*>(kZeroRecord);
                    const int g = lane ^ swz8(row);
                    if (lane < 40 && g <= 36) copy(src + g * 16, dst + row * kRec8Row);
                }
            }
        };
        auto issue = [&](int c) {
            if (c >= nch) return;
            if (kv_shared) issue_with(c, std::integral_constant<bool, true>{});
            else issue_with(c, std::integral_constant<bool, false>{});
        };

        // ---- S^T for this wave's 16 tokens of chunk c, masked and scaled, and the pair's row
        // maxima (one barrier).  Rows that see their first finite scores take the chunk maximum
        // as reference; returns whether a row outgrew its reference (a restart vote).
        auto scores = [&](int c, f4 (&s)[2], float (&mx)[2], float (&tsc)[4]) -> bool {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            const int tb = t0 + c * kChunk;
            f4 s2[2][2];                // [n][ks&1]: four independent MFMA chains
#pragma unroll
            for (int n = 0; n < 2; ++n) s2[n][0] = s2[n][1] = f4{0.f, 0.f, 0.f, 0.f};
            auto kfrag = [&](int ks) -> bf16x8 {
                if constexpr (!SPARSE) {
                    const int off = ks < 16 ? kaddr[ks & 1] + 128 * (ks >> 1) : kaddrB[ks & 1];
                    return *reinterpret_cast<const bf16x8*>(buf + off);
                } else {
                    const int gq = 2 * ks + (g4 >> 1);
                    const uint2 w = *reinterpret_cast<const uint2*>(buf + krow * kRec8Row + ((gq ^ swz8(krow)) << 4) + (g4 & 1) * 8);
                    return fp8x8_to_bf16(w.x, w.y);
                }
            };
            // fragments are read kPF steps ahead of their MFMAs: with one wave per SIMD nothing
            // else hides the LDS latency
            bf16x8 kf[kPF];
#pragma unroll
            for (int i = 0; i < kPF - 1; ++i) kf[i] = kfrag(i);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                if (ks + kPF - 1 < 18) kf[(ks + kPF - 1) % kPF] = kfrag(ks + kPF - 1);
#pragma unroll
                for (int n = 0; n < 2; ++n) s2[n][ks & 1] = mfma16(kf[ks % kPF], qf[n][ks], s2[n][ks & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) s[n] = s2[n][0] + s2[n][1];
            bool tok_ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * h + 4 * g4 + i;
                if constexpr (SPARSE) {
                    const int idx = tb + tok < t1 ? lidx[c * kChunk + tok] : -1;
                    tok_ok[i] = idx >= 0;
                    tsc[i] = idx >= 0 ? *reinterpret_cast<const float*>(buf + tok * kRec8Row + ((36 ^ swz8(tok)) << 4)) : 0.f;
                } else {
                    tok_ok[i] = tb + tok < t1;
                    tsc[i] = 1.f;
                }
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                mx[n] = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bool valid = tok_ok[i];
                    if constexpr (!SPARSE) valid = valid && (tb + 16 * h + 4 * g4 + i <= limit[n]);
                    const float f = SPARSE ? a.scale_log2 * tsc[i] : a.scale_log2;
                    s[n][i] = valid ? s[n][i] * f : -INFINITY;
                    mx[n] = fmaxf(mx[n], s[n][i]);
                }
                mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 16));
                mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 32));
                if (g4 == 0) xch[(wave * 2 + n) * 16 + l16] = mx[n];
            }
            __syncthreads();
            bool outgrown = false;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                mx[n] = fmaxf(mx[n], xch[(partner * 2 + n) * 16 + l16]);
                if (m_run[n] == -INFINITY) m_run[n] = mx[n];     // acc and l are still exactly 0
                else outgrown = outgrown || (mx[n] > m_run[n] + kRefSlack);
            }
            return __builtin_amdgcn_ballot_w64(outgrown) != 0;
        };

        // ---- P for this wave's tokens, P^T halves exchanged in the pair together with the
        // restart votes of all waves (one barrier), and O^T[256h + ..][row] += V^T P^T over the
        // chunk's 32 tokens.  Returns true (and skips P.V) when the workgroup must restart.
        auto accumulate = [&](int c, const f4 (&s)[2], const float (&tsc)[4], bool vote) -> bool {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            uint2 mine[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const float m_use = (m_run[n] == -INFINITY) ? 0.f : m_run[n];
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = exp2_fast(s[n][i] - m_use);
                    l_run[n] += p[i];
                    if constexpr (SPARSE) p[i] *= tsc[i];
                }
                mine[n] = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
                pex[(wave * 2 + n) * 64 + lane] = mine[n];
            }
            if (lane == 0) votes[wave] = vote ? 1 : 0;
            __syncthreads();
            int any = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) any |= votes[w];
            if (__builtin_amdgcn_readfirstlane(any)) return true;
            bf16x8 pT[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const uint2 other = pex[(partner * 2 + n) * 64 + lane];
                const uint4 pk = h == 0 ? make_uint4(mine[n].x, mine[n].y, other.x, other.y)
                                        : make_uint4(other.x, other.y, mine[n].x, mine[n].y);
                pT[n] = __builtin_bit_cast(bf16x8, pk);
            }
            auto vfrag = [&](int dt) -> bf16x8 {    // dt: global 16-dim tile 0..31
                if constexpr (!SPARSE) {
                    const int off = 128 * (dt >> 2);
                    const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr[0][dt & 3] + off));
                    const short4v v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr[1][dt & 3] + off));
                    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
                } else {
                    typedef int v2i __attribute__((ext_vector_type(2)));
                    const v2i w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i*)(buf + v8row * kRec8Row + ((dt ^ swz8(v8row)) << 4) + (l16 & 1) * 8));
                    return fp8x8_to_bf16((unsigned)w[0], (unsigned)w[1]);
                }
            };
            bf16x8 vf[kPF];
#pragma unroll
            for (int i = 0; i < kPF - 1; ++i) vf[i] = vfrag(16 * h + i);
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) {
                if (dt + kPF - 1 < 16) vf[(dt + kPF - 1) % kPF] = vfrag(16 * h + dt + kPF - 1);
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[dt][n] = mfma16(vf[dt % kPF], pT[n], acc[dt][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
            return false;
        };

        // ---- passes over the segment (a second one only after a restart vote).  Pipeline:
        // DEPTH-1 chunks in flight; all waves run the same barriers.
        for (;;) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                l_run[n] = 0.f;
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) acc[dt][n] = f4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int c = 0; c < DEPTH - 1; ++c) issue(c);
            bool restart = false;
            float mx[2];
            for (int k = 0; k < nch; ++k) {
                // copies are counted exactly (every chunk issues C::OPS per wave), so chunk k has
                // landed once at most DEPTH-2 later chunks' copies remain in flight
                if (k + DEPTH - 2 < nch) {
                    if constexpr (DEPTH - 2 == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DEPTH - 2) * C::OPS) : "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                __syncthreads();               // chunk k is in LDS; slot k-1 is no longer read
                issue(k + DEPTH - 1);
                f4 sc[2];
                float tsc[4];
                const bool vote = scores(k, sc, mx, tsc);
                if (accumulate(k, sc, tsc, vote)) {
                    restart = true;
                    break;
                }
            }
            if (!restart) break;
            // drain the copies in flight, then start over with each row's largest maximum so far
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
#pragma unroll
            for (int n = 0; n < 2; ++n) m_run[n] = fmaxf(m_run[n], mx[n]);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
        {
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
    hipLaunchKernelGGL((mla_decode_big_kernel<SPARSE, PAIRS>), dim3(items * R), dim3(C::WAVES * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_big(const AttnArgs& a, bool sparse, hipStream_t stream) {
    const int items = sparse ? a.batch * a.num_parts : a.num_parts;
    if (big_pairs(a.M) == 1)
        return sparse ? launch_big_t<true, 1>(a, items, stream) : launch_big_t<false, 1>(a, items, stream);
    return sparse ? launch_big_t<true, 2>(a, items, stream) : launch_big_t<false, 2>(a, items, stream);
}

}  // namespace mla
