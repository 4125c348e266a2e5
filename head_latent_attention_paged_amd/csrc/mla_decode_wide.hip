// gfx950 paged decode kernel for many query rows per KV stream, one wave per SIMD: bf16 pages
// (576- or 512-wide rows) and FP4 pages of 512-wide rows.
//
// A workgroup holds 128 query rows in four waves, one per SIMD; each wave owns 32 whole rows.
// Per 32-token chunk a wave computes S^T[32 tokens x 32 rows] = K Q^T with 32x32x16 MFMAs
// (tokens on the MFMA M side: "FlashMLA-ETAP: Efficient Transpose Attention Pipeline ...",
// section 핵심 메커니즘, transposed form), the online softmax of its rows over all 32 tokens, and
// O^T[512 dims x 32 rows] += V^T P^T.  In the 32x32 accumulator layout a lane holds 16 tokens of
// one row, so a row's maximum and sum need one lane exchange, and the lane's probabilities are
// exactly its half of the P^T B operand of the P.V MFMAs (V^T is read in the matching token
// order with transposing LDS reads).  No probability crosses a wave.  Each K or V^T fragment read
// from LDS feeds a 32-row MFMA, twice the work per LDS byte of a 16-row tile, and the 512 O^T
// accumulators of a wave's rows live in the accumulation registers.
//
// Chunk loop, iteration k: Q.K^T(k) with the copies of chunk k+3 spread over its MFMAs, the
// masking and the first token step's probabilities of chunk k, then P.V(k) with the second
// step's probabilities and the lane's maximum computed between its MFMAs.  A chunk's slot frees
// as soon as its own P.V is done, so three chunks are in flight while one is used (timing copies
// without the HBM copies ran the compute-bound shapes 17-19% faster: the kernel waits on its
// copies).  One workgroup barrier per chunk guards the ring, which all four waves fill.
//
// Softmax reference: a row's reference is the maximum of its first chunk and never moves inside
// a pass, so the accumulators are touched only by MFMAs; p = 2^(s - m) <= 2^kRefSlack keeps bf16
// P and the fp32 sums finite.  A score that outgrows its row's reference by more (or a finite
// score in a row whose first chunk had none) makes the workgroup run the pass again with each
// row's maximum over the segment as reference (at most once per segment).
//
// FP4 pages ("[flashinfer] FlashInfer, NVFP4를 활용한 DeepSeek-V4 디코딩 성능 최적화", README
// tensor table: E2M1 codes two per byte, UE4M3 scales per 16 values): each wave loads its 8 rows
// of a chunk one chunk ahead into registers and converts them exactly into the bf16 chunk layout
// (every E2M1 x UE4M3 product is a bf16 value), so the MFMA core is the bf16 one.
#include "mla_device.h"

namespace mla {

namespace wide {

typedef float f16v __attribute__((ext_vector_type(16)));

#ifndef MLA_WIDE_KPF
#define MLA_WIDE_KPF 4
#endif
#ifndef MLA_WIDE_VPF
#define MLA_WIDE_VPF 4
#endif

constexpr int kWaves = 4;
constexpr int kRowsWave = 32;
constexpr int kRowsWg = kWaves * kRowsWave;
constexpr float kRefSlack = 64.f;
// LDS chunk layout (measured conflict-free on gfx950 for both operand reads): region A holds
// dims 0..511 of a row in 1 KB at a 1088-byte row stride, its 16-byte granule g at slot
// g ^ ((row >> 2) & 3): the 32 tokens x 16 B of a K read and the 4 rows x 64 B of a V^T
// transposing read per half-wave both fall on distinct banks (at a 1056-byte stride, without the
// XOR, half the LDS cycles of this kernel were bank conflicts).  Region B holds the 64 RoPE dims
// in 128-byte rows, granule g at slot g ^ swzB(row).
constexpr int kRowA16 = 1088;
__device__ __forceinline__ int swzA(int r) { return (r >> 2) & 3; }
constexpr int kRegionB16 = kChunk * kRowA16;
constexpr int kChunk16 = kRegionB16 + kChunk * 128;

// kernel modes: bf16 pages (direct HBM -> LDS copies), and FP4 pages of the 512-wide rows, whose
// rows are gathered into registers one chunk ahead and converted exactly to bf16 in the same
// LDS layout, so the MFMA core is the same for both.  (fp8 records would need 20 more registers
// for the records in flight than this kernel has next to 576-wide Q; they use the row-split
// kernel.  The mode numbers are the row-split kernel's.)
constexpr int kPagedBf16 = 0, kPagedFp4 = 3;
// output staging: a wave's 32 rows x 1 KB (bf16 O, or half the fp32 partial) at this pitch
constexpr int kOutPitch = 1040;
__device__ __forceinline__ int swzB(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ f16v mfma32(bf16x8 a, bf16x8 b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The S^T chain with its accumulator in VGPRs (the accumulation registers hold all of O^T):
// the first step starts from zero, later steps accumulate through SrcC back to back.  The
// compiler does not see these as MFMAs, so s_result_fence waits out the result latency
// (32x32x16: 16 passes; a VALU read of the result needs 18 wait states) before anything reads S.
__device__ __forceinline__ void mfma32_v_first(f16v& c, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v(f16v& c, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void s_result_fence(f16v& c) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}

template <bool GATHER, int D>
struct Cfg {
    static constexpr int OPS = D == kDqk ? 9 : 8;          // 1 KB copies per wave per chunk
    // a ring slot: a bf16 chunk, and for gathered records their 32 token scales (fp32)
    static constexpr int BUF = kChunk16 + (GATHER ? kChunk * 4 : 0);
    // ring: chunk k (Q.K^T, then P.V) and, copied, three in flight; gathered, chunk k+1
    // (converted while chunk k+2 is loaded into registers) and a spare slot
    static constexpr int DEPTH = GATHER ? 3 : 4;
    static constexpr int AHEAD = DEPTH - 1;
    static constexpr int RING = DEPTH * BUF;
    static constexpr int PAGES = kWaves * 64 * 4;          // per-wave page windows
    static constexpr int VOTES = kWaves * 4;
    static constexpr int USED = RING + PAGES + VOTES;
    static constexpr int STAGE = kWaves * kRowsWave * kOutPitch;
    static constexpr int LDS = USED > STAGE ? USED : STAGE;
};

// D: width of a cached row, 576 (512 latent + 64 RoPE dims) or 512 (the DeepSeek-V4 latent row
// that is both K and V: bf16 or FP4 pages)
// FUSED (512-wide rows): the fused decode, whose query gets its RMS norm and rotation as it is
// loaded and whose final rows leave as FP8 codes after the conjugate rotation
template <int MODE, bool SHARED, int D, bool FUSED = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_wide_kernel(const AttnArgs a) {
    static_assert(!FUSED || D == kDv, "the fused decode works on 512-wide rows");
    constexpr bool FP4 = MODE == kPagedFp4;
    constexpr bool GATHER = FP4;
    static_assert(MODE == kPagedBf16 || (FP4 && D == kDv), "FP4 pages hold 512-wide rows");
    constexpr int KS = D / 16;                     // Q.K^T MFMA steps (16 dims each)
    constexpr int ROWB = D * 2;                    // bytes of a bf16 row in HBM
    // raw masked scores with the scale in the exponent (576-wide bf16 rows, positive scales);
    // otherwise scores are scaled before masking, which takes any scale
    constexpr bool RAWMAX = !GATHER && D == kDqk;
    using C = Cfg<GATHER, D>;
    constexpr int DEPTH = C::DEPTH, AHEAD = C::AHEAD;
    // P.V of a chunk right after its own Q.K^T (see the chunk loop), except for the fused decode
    // over FP4 pages
    constexpr bool kEarlyPV = !(GATHER && FUSED);
    // FP4 gathers per lane per chunk: a wave loads 8 rows of 16 code granules (plus 2 scale
    // bytes per granule), 128 granules in 2 loads of 64 lanes
    constexpr int NG = 2;
    constexpr unsigned REC = 256u;                 // code bytes per FP4 row
    constexpr int PF = MLA_WIDE_KPF;               // K fragment prefetch distance (MFMA steps)
    constexpr int VPF = MLA_WIDE_VPF;              // V^T fragment prefetch distance
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    // fused decode: the query-norm weight, staged once per workgroup (the prologue of every
    // segment reads it fragment by fragment)
    __shared__ __attribute__((aligned(16))) float s_qw[FUSED ? kDv : 4];
    char* ring = smem;
    int* lpages = reinterpret_cast<int*>(smem + C::RING);
    int* votes = reinterpret_cast<int*>(smem + C::RING + C::PAGES);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31;         // row of the B / C operands, token of a K read
    const int g = lane >> 5;           // k half of the operands
    const int j16 = lane & 15, ih = (lane >> 4) & 1;

    // ---- work item -> (part, row group); row groups of one part share an XCD (all but the
    // parts beyond the last multiple of 8)
    const int R = ceil_div(a.M, kRowsWg);
    const int n_items = a.num_parts;
    int item, rg;
    xcd_item(blockIdx.x, n_items, R, item, rg);

    auto copy_s = [&](const void* sbase, unsigned voff, const void* l) {
        if constexpr (SHARED) dma16_s_shared(sbase, voff, l);
        else dma16_s(sbase, voff, l);
    };

    // ---- LDS fragment offsets that do not depend on the chunk
    // K (A operand), step ks: token r32, dims 16*ks + 8*g .. +7 = granule 2ks + g.  Region A slot
    // (2ks + g) ^ swzA: bits 0 and 1 are g ^ swzA.0 and (ks & 1) ^ swzA.1, so even and odd steps
    // each have one base and a 64-byte step.  Region B (RoPE step m = ks-32): slot
    // (2m + g) ^ swzB = ((2m) ^ (swzB & 6)) | (g ^ (swzB & 1)).
    const int kaddrE = r32 * kRowA16 + 16 * ((((swzA(r32) >> 1) & 1) << 1) | (g ^ (swzA(r32) & 1)));
    const int kaddrO = r32 * kRowA16 + 16 * (((1 ^ ((swzA(r32) >> 1) & 1)) << 1) | (g ^ (swzA(r32) & 1)));
    const int kaddrB = kRegionB16 + r32 * 128 + ((g ^ (swzB(r32) & 1)) << 4);
    const int kswB = (swzB(r32) & 6) << 4;
    // V^T (A operand) of dim tile dt and token step s: the 16-lane group (ih, g) reads token rows
    // 4g + 16s + j16/4 (and +8) at dims 32*dt + 16*ih + 4*(j16 & 3); after the transpose lane
    // (dim 32*dt + r32, g) holds tokens 4g + 16s + {0..3} and 4g + 16s + 8 + {0..3}.  Those dims
    // are granule 4dt + 2ih + (j16&3)/2, byte 8*(j16&1); the rows' swzA is g (and (g+2)&3 for
    // the rows +8), which only touches the granule's low two bits.
    const int vgr = 2 * ih + ((j16 & 3) >> 1);
    const int vaddr1 = (4 * g + (j16 >> 2)) * kRowA16 + ((vgr ^ g) << 4) + (j16 & 1) * 8;
    const int vaddr2 = (4 * g + (j16 >> 2) + 8) * kRowA16 + ((vgr ^ ((g + 2) & 3)) << 4) + (j16 & 1) * 8;
    // the lane id, recomputed where it is needed (no register holds it through the loops)
    auto lane_now = []() {
        int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        asm volatile("" : "+v"(l));
        return l;
    };
    // the value of lane ^ 32 (the other half of a row)
    auto xor32 = [&](float x) {
        return __int_as_float(__builtin_amdgcn_ds_bpermute((lane_now() ^ 32) << 2, __float_as_int(x)));
    };
    // FP4 code rows and scale rows, addressed with 64-bit offsets (no limit on the cache size)
    const char* pool = static_cast<const char*>(a.kv);
    const char* pool_sc = static_cast<const char*>(a.kv_scale);

    bf16x8 qf[KS];
    f16v acc[16];
    float m_run, l_run, m_lane;

    auto run_segment = [&](int grp, int t0, int t1, int L, bool final_out, int slot) {
        const int nch = ceil_div(t1 - t0, kChunk);
        // ---- Q fragments (B operand): dims 16*ks + 8*g .. +7 of this lane's row
        {
            // per-lane addresses are built where they are used (opaque row), not held through the
            // chunk loop
            const int ql = lane_now();
            const int qrw = rg * kRowsWg + kRowsWave * wave + (ql & 31);
            const int qr = qrw < a.M ? qrw : 0, qg = ql >> 5;
            const char* qrow = static_cast<const char*>(a.q) + ((size_t)grp * a.M + qr) * ROWB + qg * 16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint4 v = *reinterpret_cast<const uint4*>(qrow + ks * 32);
                if (qrw >= a.M) v = make_uint4(0, 0, 0, 0);
                qf[ks] = __builtin_bit_cast(bf16x8, v);
            }
            if constexpr (FUSED) {
                // the query's RMS norm over its 512 dims (the lane holds dims 16ks + 8qg .. +7,
                // lane ^ 32 the other half) with the shared weight, then the rotation of the
                // pairs (448 + 2i, 449 + 2i) by the query token's angles; the result is the bf16
                // B operand
                float ss = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float f = (float)qf[ks][e];
                        ss = __builtin_fmaf(f, f, ss);
                    }
                ss += xor32(ss);
                const float rinv = 1.f / sqrtf(ss * (1.f / kDv) + a.qn_eps);
                int hq = a.h_q;
                asm volatile("" : "+s"(hq));
                const float* cs = a.rope_cs + ((size_t)grp * a.s_q + qr / hq) * 64;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    // (opaque: the sum of squares above does not keep its 256 floats live for this)
                    asm volatile("" : "+v"(qf[ks]));
                    const int d0 = 16 * ks + 8 * qg;
                    const f4 w0 = *reinterpret_cast<const f4*>(s_qw + d0);
                    const f4 w1 = *reinterpret_cast<const f4*>(s_qw + d0 + 4);
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (float)qf[ks][e] * rinv * (e < 4 ? w0[e] : w1[e - 4]);
                    if (16 * ks >= kRopeStart) {
                        const int i0 = (d0 - kRopeStart) >> 1;
                        const f4 c = *reinterpret_cast<const f4*>(cs + i0);
                        const f4 sn = *reinterpret_cast<const f4*>(cs + 32 + i0);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float x = v[2 * j], y = v[2 * j + 1];
                            v[2 * j] = x * c[j] - y * sn[j];
                            v[2 * j + 1] = x * sn[j] + y * c[j];
                        }
                    }
                    const uint4 u = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
                    qf[ks] = __builtin_bit_cast(bf16x8, u);
                    // one fragment at a time: the weight loads are not hoisted ahead of the loop
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        m_run = -INFINITY;
        // the lane's tokens are visible below this position (past the segment's end, or the
        // causal limit of the row), relative to its token offset 4*g in a chunk
        const int vl = lane_now();
        const int vrow = rg * kRowsWg + kRowsWave * wave + (vl & 31), vg = vl >> 5;
        int hq = a.h_q;                    // (the divisor's reciprocal is not held either)
        asm volatile("" : "+s"(hq));
        const int vis_end = min(t1, (a.causal ? (L - a.s_q + vrow / hq) : (L - 1)) + 1) - 4 * vg;

        // page numbers of the segment, 64 at a time into a per-wave LDS window
        int bt_base = -1000000;
        auto page_of = [&](int p) {
            int* win = lpages + wave * 64;
            if (p - bt_base >= 64 || p < bt_base) {
                bt_base = p;
                const int np = ceil_div(t1, kPage) - (t0 >> 6);
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int v = (ln < np - p) ? a.block_table[(size_t)grp * a.max_blocks + (t0 >> 6) + p + ln] : 0;
                win[ln] = v;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            return __builtin_amdgcn_readfirstlane(win[p - bt_base]);
        };

        // ---- copies of one chunk: 32 rows of region A (1 KB each) and, for 576-wide rows, 4 KB of
        // region B (8 rows of 128 B per copy), spread over the four waves.  Chunks past the
        // segment's end re-copy its last chunk into their (unused) slot, so the number of copies
        // per chunk is fixed and the waits are exact.
        struct Plan {
            const char* base;
            char* dst;
            int nrows;
        };
        auto plan_for = [&](int c) {
            Plan p;
            const int cc = min(c, nch - 1);
            p.dst = ring + (c % DEPTH) * C::BUF;
            const int tb = t0 + cc * kChunk;
            p.nrows = min(kChunk, t1 - tb);
            const int page = page_of(cc >> 1);
            p.base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * ROWB;
            return p;
        };
        auto copy_op = [&](const Plan& p, int j) {
            if (j < kChunk / kWaves) {        // row q = wave + 4j of region A (swzA(q) = j & 3)
                const int q = wave + kWaves * j;
                const int rr = min(q, p.nrows - 1);
                copy_s(p.base + rr * ROWB, (unsigned)(lane ^ (j & 3)) << 4, p.dst + q * kRowA16);
            } else {                          // region B rows 8*wave .. +7
                const int sl = wave * 64 + lane;
                const int br = sl >> 3;
                const int rr = min(br, p.nrows - 1);
                copy_s(p.base, (unsigned)(rr * ROWB + (64 + ((sl & 7) ^ swzB(br))) * 16),
                       p.dst + kRegionB16 + wave * 1024);
            }
        };
        auto wait_chunk = [&]() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"((AHEAD - 1) * C::OPS) : "memory"); };

        // ---- FP4 rows: load i of chunk c into registers, and its conversion into chunk c's ring
        // slot.  Load i of lane (r4 = lane >> 4, gran = lane & 15) is code granule gran of row
        // rt = 8*wave + 4i + r4 of the chunk.  swzA(rt) = (2*wave + i) & 3 is wave-uniform, so the
        // converted granule 4*gran + w lands at the lane's base cbase plus a wave-uniform offset.
        // Chunks past the segment's end gather its last chunk again (into an unused slot).
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        u32x4 gv[GATHER ? NG : 1];
        unsigned g_bad = 0;       // bit i: load i of this lane reads no record (unused entry)
        unsigned short g_sc[FP4 ? NG : 1];      // FP4: the two scale bytes of the lane's granule
        unsigned gp_rec0 = 0;     // row of the chunk's first token (wave-uniform)
        int gp_n = 0;             // tokens of the chunk that are read (0: page outside the cache)
        unsigned chunk_ok = 0;    // bit c & 3: chunk c's page lies in the cache (wave-uniform)
        auto gather = [&](int c, int i) {
            const int cc = min(c, nch - 1);
            const int ln = lane_now();
            const int rt = 4 * i + (ln >> 4), gran = ln & 15;    // row within the wave's 8
            // a chunk lies inside one page (segments start on a page); gather 0 comes first
            if (i == 0) {
                const int tb = t0 + cc * kChunk;
                const int pg = page_of(cc >> 1);
                const bool pg_ok = pg >= 0 && (long long)pg * kPage < a.kv_rows;
                gp_rec0 = (unsigned)pg * kPage + (tb & 63) + 8 * wave;
                gp_n = pg_ok ? min(kChunk, t1 - tb) - 8 * wave : 0;
                chunk_ok = (chunk_ok & ~(1u << (c & 3))) | ((pg_ok ? 1u : 0u) << (c & 3));
            }
            // an unused token reads row 0 (converted to zeros below)
            const bool bad = rt >= gp_n;
            const size_t rec = bad ? 0 : (size_t)(gp_rec0 + rt);
            g_bad = (g_bad & ~(1u << i)) | ((bad ? 1u : 0u) << i);
            const u32x4* gp = reinterpret_cast<const u32x4*>(pool + rec * REC + gran * 16);
            if constexpr (SHARED) gv[i] = *gp;
            else gv[i] = __builtin_nontemporal_load(gp);
            g_sc[i] = *reinterpret_cast<const unsigned short*>(pool_sc + rec * 32 + gran * 2);
        };
        // FP4: quarter w (8 values: granule 4*gran + w of the bf16 row) of load i; the block scale
        // multiplies in fp32 after an exact unit-scale conversion (the product is a bf16 value);
        // the token entry is 1, or NaN for an unused one
        auto convert_fp4 = [&](int c, int i, int w) {
            const int ln = lane_now();
            // (a 24-bit multiply: full rate, where a 32-bit one issues at a quarter)
            const int cbase = (int)__umul24((unsigned)(ln >> 4), (unsigned)kRowA16) + (ln & 15) * 64;
            char* slot = ring + (c % DEPTH) * C::BUF + (8 * wave + 4 * i) * kRowA16 + ((w ^ ((2 * wave + i) & 3)) << 4);
            // an unused token converts to zeros (row 0's bytes, which it read, are not its own);
            // the scale is converted in every lane and then masked, without a branch
            const bool none = (g_bad >> i) & 1;
            const unsigned codes = none ? 0u : gv[i][w];
            const float sc_all = __builtin_amdgcn_cvt_f32_fp8((int)((unsigned)g_sc[i] >> (8 * (w >> 1))), 0);
            const float sc = __uint_as_float(__float_as_uint(sc_all) & (none ? 0u : ~0u));
            unsigned o[4];
#define MLA_FP4_PAIR(B_)                                                              \
    {                                                                                 \
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, B_);     \
        o[B_] = pack_bf16x2(v[0] * sc, v[1] * sc);                                    \
    }
            MLA_FP4_PAIR(0) MLA_FP4_PAIR(1) MLA_FP4_PAIR(2) MLA_FP4_PAIR(3)
#undef MLA_FP4_PAIR
            *reinterpret_cast<uint4*>(slot + cbase) = make_uint4(o[0], o[1], o[2], o[3]);
            if (w == 0 && (ln & 15) == 0)
                *reinterpret_cast<unsigned*>(ring + (c % DEPTH) * C::BUF + kChunk16 + (8 * wave + 4 * i + (ln >> 4)) * 4) =
                    (g_bad >> i) & 1 ? 0x7fc00000u : 0x3f800000u;
        };
        // all of chunk c's loads (prologue)
        auto convert_all = [&](int c) {
#pragma unroll
            for (int i = 0; i < NG; ++i) {
#pragma unroll
                for (int w = 0; w < 4; ++w) convert_fp4(c, i, w);
            }
        };
        // during the Q.K^T steps of a chunk: chunk cn's conversion in four quarters per load, then
        // chunk cn+1's load into the same registers
        auto gather_side = [&](int cn, int ks) {
            const int i = ks >> 3, st = ks & 7;
            if (i < NG) {
                if ((st & 1) == 1) convert_fp4(cn, i, st >> 1);
                if (st == 7) gather(cn + 1, i);
            }
        };

        // ---- LDS fragments
        auto kfrag = [&](const char* buf, int ks) -> bf16x8 {
            const int off = ks < 32 ? ((ks & 1) ? kaddrO : kaddrE) + 64 * (ks >> 1)
                                    : kaddrB + ((32 * (ks - 32)) ^ kswB);
            return *reinterpret_cast<const bf16x8*>(buf + off);
        };
        auto vfrag = [&](const char* buf, int i) -> bf16x8 {     // i = 2 * dt + s
            const int off = 64 * (i >> 1) + 16 * kRowA16 * (i & 1);
            const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr1 + off));
            const short4v v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr2 + off));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
        };

        // S^T of chunk c for this wave's 32 rows: one accumulation chain (back-to-back MFMAs
        // accumulate through SrcC); side(ks) runs between the steps
        auto qk = [&](int c, f16v& sacc, auto&& side) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            bf16x8 kf[PF];
#pragma unroll
            for (int i = 0; i < PF - 1; ++i) kf[i] = kfrag(buf, i);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + PF - 1 < KS) kf[(ks + PF - 1) % PF] = kfrag(buf, ks + PF - 1);
                if (ks == 0) mfma32_v_first(sacc, kf[0], qf[0]);
                else mfma32_v(sacc, kf[ks % PF], qf[ks]);
                side(ks);
            }
            s_result_fence(sacc);
        };
        // O^T += V^T P^T over chunk c: token step s (16 tokens) for all 16 dim tiles, s = 0, 1
        // (the two steps of a tile are 16 MFMAs apart); side(i) runs between the MFMAs
        auto vidx = [](int n) { return 2 * (n & 15) + (n >> 4); };     // MFMA n: tile n&15, step n>>4
        // the first VPF-1 V^T fragments of chunk c's P.V (issued ahead of it)
        auto pv_head = [&](int c, bf16x8 (&vf)[VPF]) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
#pragma unroll
            for (int i = 0; i < VPF - 1; ++i) vf[i] = vfrag(buf, vidx(i));
        };
        auto pv_body = [&](int c, bf16x8 (&vf)[VPF], bf16x8 (&pb)[2], auto&& side) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
#pragma unroll
            for (int n = 0; n < 32; ++n) {
                if (n + VPF - 1 < 32) vf[(n + VPF - 1) % VPF] = vfrag(buf, vidx(n + VPF - 1));
                acc[n & 15] = mfma32(vf[n % VPF], pb[n >> 4], acc[n & 15]);
                side(n);
            }
        };
        auto pv = [&](int c, bf16x8 (&pb)[2], auto&& side) {
            bf16x8 vf[VPF];
            pv_head(c, vf);
            pv_body(c, vf, pb, side);
        };

        // ---- masking of chunk c: lane value v is token 8*(v>>2) + 4*g + (v&3) of this lane's row
        // (ROWMAX: also the row's largest masked score over both lanes, for chunk 0's reference)
        auto mask = [&](int c, f16v& s, float& mx, auto rowmax_c) {
            constexpr bool ROWMAX = decltype(rowmax_c)::value;
            const int tb = t0 + c * kChunk;
            const int bnd = vis_end - tb;                             // valid: 8*(v>>2) + (v&3) < bnd
            float m = -INFINITY;
            const bool whole = __builtin_amdgcn_ballot_w64(bnd < kChunk - 4) == 0;   // lane's last token: kChunk - 5
            if (GATHER && whole && ((chunk_ok >> (c & 3)) & 1)) {
                // every token of the chunk is read and visible to every row of the wave
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    s[v] *= a.scale_log2;
                    m = fmaxf(m, s[v]);
                }
            } else if constexpr (GATHER) {
                // token entries of the lane's tokens 8q + 4g + (0..3): NaN marks an unused one
                const char* buf = ring + (c % DEPTH) * C::BUF + kChunk16 + 16 * g;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f4 sc = *reinterpret_cast<const f4*>(buf + 32 * q);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int v = 4 * q + r;
                        const bool ok = (sc[r] == sc[r]) & (8 * q + r < bnd);
                        s[v] = ok ? s[v] * a.scale_log2 : -INFINITY;
                        m = fmaxf(m, s[v]);
                    }
                }
            } else if (whole) {
                // every token of the chunk is visible to every row of the wave: no mask
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if constexpr (!RAWMAX) s[v] *= a.scale_log2;
                    m = fmaxf(m, s[v]);
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const bool ok = 8 * (v >> 2) + (v & 3) < bnd;
                    if constexpr (RAWMAX) s[v] = ok ? s[v] : -INFINITY;
                    else s[v] = ok ? s[v] * a.scale_log2 : -INFINITY;
                    m = fmaxf(m, s[v]);
                }
            }
            if constexpr (ROWMAX) {
                if constexpr (RAWMAX) m *= a.scale_log2;   // a positive scale commutes with the max
                m = fmaxf(m, xor32(m));
                mx = m;
            }
        };
        // probabilities under the row's reference of token step h2 (lane values 8*h2 .. +7): the
        // bf16 B operand of that step of P.V
        // (mx: the running maximum of the masked scores taken)
        auto probs = [&](int c, const f16v& s, int h2, float& mx) -> bf16x8 {
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = s[8 * h2 + e];
                mx = fmaxf(mx, x);
                if constexpr (RAWMAX) p[e] = exp2_fast(__builtin_fmaf(x, a.scale_log2, -m_use));
                else p[e] = exp2_fast(x - m_use);
                l_run += p[e];
            }
            const uint4 u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                       pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
            return __builtin_bit_cast(bf16x8, u);
        };
        auto no_side = [](int) {};

        // ---- passes over the segment (a second one only after a restart vote)
        for (int pass = 0;; ++pass) {
            l_run = 0.f;
            m_lane = -INFINITY;
#pragma unroll
            for (int t = 0; t < 16; ++t) acc[t] = f16v{};
            bool outgrown = false;
            if constexpr (!GATHER) {
#pragma unroll
                for (int c = 0; c < AHEAD; ++c) {
                    const Plan p = plan_for(c);
#pragma unroll
                    for (int j = 0; j < C::OPS; ++j) copy_op(p, j);
                }
                wait_chunk();
            } else {
#pragma unroll
                for (int i = 0; i < NG; ++i) gather(0, i);
                convert_all(0);
#pragma unroll
                for (int i = 0; i < NG; ++i) gather(1, i);
            }
            __syncthreads();
            // one chunk after its Q.K^T: masking, the probabilities of token step 0, then P.V of
            // the chunk with step 1's probabilities and the lane's largest masked score computed
            // between its MFMAs.  The row's reference comes from chunk 0 (a restart pass keeps
            // its own), so a later chunk's probabilities need no maximum of their own; its lane
            // maximum feeds the restart vote and reference (the row's is taken at the restart).
            auto finish = [&](int c, f16v& s, auto first_c) {
                constexpr bool FIRST = decltype(first_c)::value;
                // bf16 pages: the first V^T reads of the chunk's P.V go out before the masking and
                // the probabilities, whose VALU work then covers their latency (FP4 pages measured
                // slower that way: their conversion work sits between the same MFMAs)
                bf16x8 vf[VPF];
                if constexpr (!GATHER) pv_head(c, vf);
                float mx = 0.f;
                mask(c, s, mx, std::integral_constant<bool, FIRST>{});
                if constexpr (FIRST) {
                    m_lane = fmaxf(m_lane, mx);
                    if (m_run == -INFINITY) m_run = mx;
                }
                bf16x8 pb[2];
                float ml = -INFINITY;
                pb[0] = probs(c, s, 0, ml);
                if constexpr (GATHER) pv_head(c, vf);
                pv_body(c, vf, pb, [&](int n) {
                    if (n == 2) pb[1] = probs(c, s, 1, ml);
                });
                if constexpr (!FIRST) {
                    if constexpr (RAWMAX) ml *= a.scale_log2;   // a positive scale commutes with the max
                    m_lane = fmaxf(m_lane, ml);
                    // also true for a finite score in a row without a reference
                    outgrown = outgrown | (ml > m_run + kRefSlack);
                }
            };
            if constexpr (kEarlyPV) {
                // chunk 0: Q.K^T with the copies of chunk AHEAD (gathered: the conversion of chunk 1
                // and the loads of chunk 2) spread over it, then its reference, probabilities and P.V
                {
                    f16v s;
                    if constexpr (!GATHER) {
                        const Plan p = plan_for(AHEAD);
                        qk(0, s, [&](int ks) {
                            if ((ks & 3) == 1 && ks / 4 < C::OPS) copy_op(p, ks / 4);
                        });
                    } else {
                        qk(0, s, [&](int ks) { gather_side(1, ks); });
                    }
                    finish(0, s, std::true_type{});
                }
                for (int k = 1; k < nch; ++k) {
                    if constexpr (!GATHER) wait_chunk();
                    // chunk k in LDS for every wave; the slot of chunk k-1, whose P.V every wave has
                    // done, free for the copies of chunk k+AHEAD (gathered: slot (k+1) % DEPTH, for the
                    // conversion of chunk k+1)
                    __syncthreads();
                    f16v s;
                    if constexpr (!GATHER) {
                        const Plan p = plan_for(k + AHEAD);
                        qk(k, s, [&](int ks) {
                            if ((ks & 3) == 1 && ks / 4 < C::OPS) copy_op(p, ks / 4);
                        });
                    } else {
                        qk(k, s, [&](int ks) { gather_side(k + 1, ks); });
                    }
                    finish(k, s, std::false_type{});
                }
            } else {
                // (the fused decode over FP4 pages, whose registers do not fit the order above:
                // P.V(k-1) runs after Q.K^T(k), with chunk k's masking and probabilities spread
                // over its MFMAs)
                bf16x8 pb[2];
                {
                    f16v s;
                    qk(0, s, [&](int ks) { gather_side(1, ks); });
                    float mx, ml = -INFINITY;
                    mask(0, s, mx, std::true_type{});
                    m_lane = fmaxf(m_lane, mx);
                    if (m_run == -INFINITY) m_run = mx;
                    pb[0] = probs(0, s, 0, ml);
                    pb[1] = probs(0, s, 1, ml);
                }
                for (int k = 1; k < nch; ++k) {
                    __syncthreads();
                    f16v s;
                    qk(k, s, [&](int ks) { gather_side(k + 1, ks); });
                    float mx = 0.f, ml = -INFINITY;
                    pv(k - 1, pb, [&](int n) {
                        if (n == 3) {
                            mask(k, s, mx, std::true_type{});
                            m_lane = fmaxf(m_lane, mx);
                            // also true for a finite score in a row without a reference
                            outgrown = outgrown | (mx > m_run + kRefSlack);
                        }
                        if (n == 16) pb[0] = probs(k, s, 0, ml);
                    });
                    pb[1] = probs(k, s, 1, ml);
                }
                pv(nch - 1, pb, no_side);
            }
            // the copies past the segment's end land; every wave's vote visible
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // (the ballot runs on the whole wave: inside the lane-0 branch it would see one row)
            const bool wave_vote = __builtin_amdgcn_ballot_w64(outgrown) != 0;
            if (lane == 0) votes[wave] = wave_vote ? 1 : 0;
            __syncthreads();
            int any = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) any |= votes[w];
            // (a second pass, whose reference is the segment maximum, cannot vote; the bound on
            // the passes is a guard)
            if (__builtin_amdgcn_readfirstlane(any) == 0 || pass == 1) break;
            // run the pass again with each row's maximum over the segment as reference
            m_run = fmaxf(m_lane, xor32(m_lane));
            __syncthreads();               // votes read before the next pass writes them
        }

        // ---- row sums: the two lanes of a row
        l_run += xor32(l_run);
        float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
        const int el = lane_now();
        const int orow = rg * kRowsWg + kRowsWave * wave + (el & 31);
        if (final_out && a.sinks) {
            // the head's attention sink joins the denominator (a split row gets it in the combine)
            int hs = a.h_q;
            asm volatile("" : "+s"(hs));
            const float sk = a.sinks[(orow < a.M ? orow : 0) % hs];
            const float hi = fmaxf(lse_v, sk), lo = fminf(lse_v, sk);
            const float tot = lo == -INFINITY ? hi : hi + log1pf(expf(lo - hi));
            inv *= l_run > 0.f ? expf(lse_v - tot) : 0.f;
            lse_v = tot;
        }
        if (orow < a.M && el < 32) {
            if (final_out) a.lse[(size_t)grp * a.M + orow] = lse_v;
            else a.part_lse[(size_t)slot * a.M + orow] = lse_v;
        }
        // ---- output through LDS: each half of the wave's O (32 rows x 256 dims, fp32 x 1/l) goes
        // to its own staging area, then out as whole rows: bf16 O, or the fp32 partial.  One
        // path for both, tile by tile.  Lane value v of dim tile dt is dim 32*dt + 8*(v>>2) +
        // 4*g + (v&3).
        char* stg = smem + wave * (kRowsWave * kOutPitch);
        const int row0 = rg * kRowsWg + kRowsWave * wave;
        // computed here, not hoisted out of the segment and pass loops, where they would hold
        // registers through the chunk loop
        int nrow = a.M - row0;
        asm volatile("" : "+s"(nrow));
        const int ln = el, er = el & 31, eg = el >> 5;
        __syncthreads();                   // the ring is no longer read: LDS is free
        if (FUSED && final_out) {
            // the conjugate rotation of dims 448..511 (tiles 14 and 15) by the query token's
            // angles, then the FP8 cast with one scale per row (amax / 448): codes through LDS,
            // out as whole 512-byte rows.  Lane value 4q + r of tile dt is dim 32dt + 8q + 4eg + r.
            int hq = a.h_q;
            asm volatile("" : "+s"(hq));
            const float* cs = a.rope_cs + ((size_t)grp * a.s_q + (orow < a.M ? orow : 0) / hq) * 64;
            // (the two passes below each rebuild the values from the accumulators: inv is made
            // opaque per pass, so that no pass keeps 256 products live for the other)
            auto outval = [&](int dt, int q, float (&x)[4], float iv) {
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = acc[dt][4 * q + r] * iv;
                if (32 * dt >= kRopeStart) {
                    const int i0 = (32 * dt + 8 * q + 4 * eg - kRopeStart) >> 1;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float c = cs[i0 + j], sn = cs[32 + i0 + j];
                        const float u = x[2 * j], w = x[2 * j + 1];
                        x[2 * j] = u * c + w * sn;
                        x[2 * j + 1] = w * c - u * sn;
                    }
                }
            };
            float amax = 0.f;
            float inv1 = inv;
            asm volatile("" : "+v"(inv1));
#pragma unroll
            for (int dt = 0; dt < 16; ++dt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float x[4];
                    outval(dt, q, x, inv1);
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
                    __builtin_amdgcn_sched_barrier(0);
                }
            amax = fmaxf(amax, xor32(amax));
            const float fscale = fmaxf(amax, 1.17549435e-38f) / kE4m3Max;
            const float finv = 1.f / fscale;
            float inv2 = inv;
            asm volatile("" : "+v"(inv2));
#pragma unroll
            for (int dt = 0; dt < 16; ++dt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float x[4];
                    outval(dt, q, x, inv2);
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = fminf(fmaxf(x[r] * finv, -kE4m3Max), kE4m3Max);
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
                    *reinterpret_cast<int*>(stg + er * kOutPitch + 32 * dt + 8 * q + 4 * eg) = w;
                    __builtin_amdgcn_sched_barrier(0);
                }
            if (orow < a.M && el < 32) a.out_scale[(size_t)grp * a.M + orow] = fscale;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own staging writes
            char* obase = static_cast<char*>(a.out) + ((size_t)grp * a.M + row0) * kDv;
#pragma unroll 4
            for (int i = 0; i < kRowsWave / 2; ++i) {
                const int r = 2 * i + (ln >> 5), cgr = ln & 31;
                const uint4 v = *reinterpret_cast<const uint4*>(stg + r * kOutPitch + cgr * 16);
                if (r < nrow) *reinterpret_cast<uint4*>(obase + (size_t)r * kDv + cgr * 16) = v;
            }
            __syncthreads();               // LDS free for the next segment
            return;
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const f16v& o = acc[8 * hf + dt];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f4*>(stg + er * kOutPitch + (32 * dt + 8 * q + 4 * eg) * 4) =
                        f4{o[4 * q] * inv, o[4 * q + 1] * inv, o[4 * q + 2] * inv, o[4 * q + 3] * inv};
                __builtin_amdgcn_sched_barrier(0);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own staging writes
            // bf16 rows: the output, or a split's partial (O of the split, normalised by its own
            // sum), whose LSE stays fp32 (the partials of 128-row groups are large: bf16 halves
            // the bytes the combine moves)
            char* obase = final_out ? static_cast<char*>(a.out) + ((size_t)grp * a.M + row0) * (kDv * 2) + 512 * hf
                                    : reinterpret_cast<char*>(a.part_o) + ((size_t)slot * a.M + row0) * (kDv * 2) + 512 * hf;
#pragma unroll 4
            for (int r = 0; r < kRowsWave; ++r) {
                const f4 v = *reinterpret_cast<const f4*>(stg + r * kOutPitch + ln * 16);
                if (r < nrow)
                    *reinterpret_cast<uint2*>(obase + (size_t)r * (kDv * 2) + ln * 8) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read back before the next half
        }
        __syncthreads();                   // LDS free for the next segment
    };

    {
        if constexpr (FUSED) {
            for (int i = threadIdx.x; i < kDv; i += kWaves * 64) s_qw[i] = a.qn_weight[i];
            __syncthreads();
        }
        const int* meta = a.tile_meta + (size_t)item * kMetaInts;
        const int b0 = meta[0], blk0 = meta[1], b1 = meta[2], blk1 = meta[3], slot0 = meta[4];
        for (int bb = b0; bb <= b1 && bb < a.batch; ++bb) {
            // the length and the split count in one memory round trip
            const int L = a.seqlens[bb];
            const int ns0 = a.num_splits[bb], ns1 = a.num_splits[bb + 1];
            const int nb = ceil_div(L, kPage);
            const int lo = (bb == b0) ? blk0 : 0;
            const int hi = (bb == b1) ? blk1 : nb;
            if (lo >= hi) continue;
            run_segment(bb, lo * kPage, min(hi * kPage, L), L, ns1 - ns0 == 1, (bb == b0) ? slot0 : ns0);
        }
    }
}

}  // namespace wide

hipError_t launch_decode_wide(const AttnArgs& a, hipStream_t stream) {
    const int R = (a.M + wide::kRowsWg - 1) / wide::kRowsWg;
    const dim3 grid(a.num_parts * R), block(wide::kWaves * 64);
#define MLA_WIDE_LAUNCH_F(MODE_, D_, F_)                                                                           \
    if (R > 1) hipLaunchKernelGGL((wide::mla_decode_wide_kernel<MODE_, true, D_, F_>), grid, block, 0, stream, a); \
    else hipLaunchKernelGGL((wide::mla_decode_wide_kernel<MODE_, false, D_, F_>), grid, block, 0, stream, a);
#define MLA_WIDE_LAUNCH(MODE_, D_) MLA_WIDE_LAUNCH_F(MODE_, D_, false)
    if (a.kv_fp8) return hipErrorInvalidValue;      // (the row-split kernel's mode)
    if (a.fused) {
        if (a.d_qk != kDv) return hipErrorInvalidValue;
        if (a.kv_fp4) {
            MLA_WIDE_LAUNCH_F(wide::kPagedFp4, kDv, true)
        } else {
            MLA_WIDE_LAUNCH_F(wide::kPagedBf16, kDv, true)
        }
        return hipGetLastError();
    }
    if (a.kv_fp4) {
        MLA_WIDE_LAUNCH(wide::kPagedFp4, kDv)
    } else if (a.d_qk == kDv) {
        MLA_WIDE_LAUNCH(wide::kPagedBf16, kDv)
    } else {
        MLA_WIDE_LAUNCH(wide::kPagedBf16, kDqk)
    }
#undef MLA_WIDE_LAUNCH
#undef MLA_WIDE_LAUNCH_F
    return hipGetLastError();
}

}  // namespace mla
