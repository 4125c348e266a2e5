// gfx950 decode kernel for many query rows per KV stream: paged s_q*h_q > 32, sparse h_q > 32.
//
// A workgroup holds 64 query rows in eight waves, two per SIMD, so that one wave's LDS, MFMA and
// barrier latencies overlap with the other's work.  Waves w and w^4 share 16 rows (row block
// w & 3) and split the work of a 32-token chunk between them: wave half h = w >> 2 computes
// S^T = K Q^T for tokens 16h..16h+15 (tokens on the MFMA M side, "FlashMLA-ETAP: Efficient
// Transpose Attention Pipeline ...", section 핵심 메커니즘, transposed form) and the online
// softmax of that tile, then O^T += V^T P^T for value dims 256h..256h+255 over all 32 tokens.
// The 16-token S^T tile holds, lane by lane, exactly half of the P^T elements this lane feeds
// to the 16x16x32 P.V MFMA (with V^T read in the matching token order); the other half comes
// from the partner wave through LDS.  The two value halves split the output as the pages'
// design splits it across two warpgroups.
//
// Chunk loop, iteration k: Q.K^T(k) of the own tile (the copies of a later chunk spread over
// it), then P.V(k-1) with P(k-1) from both waves while S^T(k) is masked and turned into
// probabilities, which go to LDS for the partner.  One workgroup barrier per chunk guards the
// shared ring of KV chunks and the exchanged probabilities.
//
// Softmax reference: a row's reference is the maximum of its first chunk (both tiles, which
// each wave of the pair computes for that chunk, so the two agree bit for bit) and never moves
// inside a pass, so the accumulators are touched only by MFMAs.  p = 2^(s - m) <= 2^kRefSlack
// keeps bf16 P and the fp32 sums finite; a score that outgrows its row's reference by more
// (or a finite score in a row whose first chunk had none) makes the workgroup finish the pass,
// discard it and run it again with the row's maximum over the whole segment as reference (so
// at most once per segment).
//
// Sparse fp8: a chunk is 32 gathered records ("deepseek-ai/FlashMLA" project summary, section
// 기술적 세부 사항: fp8 values plus a per-token scale, -1 = unused index).  The workgroup loads
// each record once into registers (64-bit record addresses; an unused entry reads record 0 and
// converts to zeros), converts the e4m3 codes exactly to bf16 and stores them in the same LDS
// layout as a paged chunk, so the Q.K^T / P.V core is the paged one; the token scale multiplies
// the score and the probability before P.V.
//
// FP4 pages (DeepSeek-V4 geometry, "[flashinfer] FlashInfer, NVFP4를 활용한 DeepSeek-V4 디코딩
// 성능 최적화", README tensor table): a token's 512-wide latent row is 256 bytes of E2M1 codes
// (two per byte, low nibble first) in one tensor and 32 UE4M3 scales, one per 16 values, in
// another.  The same gather path loads a row's codes (one 16-byte load per lane) and its two
// scale bytes, and writes e2m1 * scale as bf16 (exact: at most 6 significant bits) into the
// paged chunk layout.
#include "mla_device.h"

#include <type_traits>

namespace mla {

namespace rows {

constexpr int kWaves = 8;
constexpr int kRowsWg = 64;
// LDS fragment prefetch distances (MFMA steps) of the K and the V^T reads
#ifndef MLA_ROWS_KPF
#define MLA_ROWS_KPF 4
#endif
#ifndef MLA_ROWS_VPF
#define MLA_ROWS_VPF 4
#endif
constexpr int kPF = MLA_ROWS_KPF;
constexpr int kVPF = MLA_ROWS_VPF;
constexpr float kRefSlack = 64.f;

// LDS layouts, chosen by measuring the decode kernels' read patterns on gfx950 (64 banks):
// bf16 region A holds dims 0..511 of a row in 1 KB at a 1056-byte row stride, unswizzled: the
// 16 rows x 64 B of a K read (ds_read_b128) and the 8 rows x 32 B of a V^T transposing read both
// run conflict-free (at a 1024-byte stride every XOR swizzle tried left the K read at half rate).
// Region B (the 64 RoPE dims, 128 B rows): slot = granule ^ swzB(r).
constexpr int kRowA16 = 1056;
constexpr int kRegionB16 = kChunk * kRowA16;
constexpr int kChunk16 = kRegionB16 + kChunk * 128;
__device__ __forceinline__ int swzB(int r) { return (r >> 1) & 7; }

// Sparse gathers: a chunk's 32 records are 32 x 36 granules of 16 codes plus 32 scale granules;
// a wave loads 4 records as 296 half-granules of 8 bytes with 5 loads of 64 lanes (slots
// 296..319 repeat slots 232..255: same data to the same place).  Consecutive lanes hold
// consecutive half-granules, so their 16-byte bf16 conversions land side by side in LDS (whole
// granules per lane wrote 32-byte-strided halves, and a fifth of the kernel's LDS cycles were
// bank conflicts).  Index entries become record numbers once per segment;
// an unused entry (or one past the list) becomes -1, which reads record 0 and is marked unused.
// Loads take 64-bit addresses, so the record pool has no size limit.
constexpr int kGather = 5;
// output staging: a wave's 16 rows x 256 values (fp32 1 KB, bf16 512 B per row) at this row pitch
constexpr int kOutPitch = 1040;

template <bool GATHER, bool SPARSE, int D>
struct Cfg {
    // a ring slot holds a bf16 chunk; sparse adds the 32 token scales (32-byte stride)
    static constexpr int BUF = kChunk16 + (GATHER ? kChunk * 32 : 0);
    // ring slots: chunk k-1 (P.V), chunk k (Q.K^T) and, paged, AHEAD chunks in flight; sparse,
    // chunk k+1, converted while chunk k+2 is gathered into registers
    static constexpr int DEPTH = GATHER ? 3 : 4;
    static constexpr int AHEAD = DEPTH - 2;
    // paged copies per wave per chunk: 32 rows of region A + 4 KB of region B = 36 x 1 KB over
    // eight waves, the last four repeated; 512-wide rows have no region B: 32 x 1 KB
    static constexpr int OPS = D == kDqk ? 5 : 4;
    static constexpr int RING = DEPTH * BUF;
    static constexpr int IDX = SPARSE ? kMaxSparseSplit * 4 : 0;        // a split's index list
    static constexpr int PAGES = SPARSE ? 0 : kWaves * 64 * 4;            // per-wave page windows
    static constexpr int PX = 2 * kWaves * 64 * 8;                        // exchanged P, by chunk parity
    static constexpr int VOTES = 2 * kWaves * 4;                          // restart votes, by chunk parity
    static constexpr int USED = RING + IDX + PAGES + PX + VOTES;
    // the epilogue stages the output through all of LDS
    static constexpr int LDS = USED > kWaves * 16 * kOutPitch ? USED : kWaves * 16 * kOutPitch;
};

// kernel modes: bf16 pages (direct copies), sparse fp8 records through an index list, fp8 pages
// (their records gathered through an index list built from the block table), FP4 pages of the
// 512-wide rows (gathered the same way)
constexpr int kPagedBf16 = 0, kSparseFp8 = 1, kPagedFp8 = 2, kPagedFp4 = 3;
// FP4 rows: 256 code bytes (16 granules) and 32 scale bytes per token; a wave's 4 records of a
// chunk are its 64 lanes' code granules
constexpr int kFp4RowBytes = 256;
constexpr int kFp4ScaleShift = 3;     // scale offset = code offset / 8

// D: width of a cached row, 576 (512 latent + 64 RoPE dims) or 512 (the DeepSeek-V4 latent row
// that is both K and V: bf16 or FP4 pages)
template <int MODE, bool SHARED, int D = kDqk>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode_rows_kernel(const AttnArgs a) {
    constexpr bool SPARSE = MODE == kSparseFp8;
    constexpr bool GATHER = MODE != kPagedBf16;     // records gathered through the index list
    constexpr bool FP4 = MODE == kPagedFp4;
    static_assert(FP4 ? D == kDv : (D == kDqk || (D == kDv && MODE == kPagedBf16)),
                  "512-wide rows: bf16 or FP4 pages; FP4 pages: 512-wide rows");
    constexpr int NG = FP4 ? 1 : kGather;            // gather loads per lane per chunk
    constexpr unsigned REC = FP4 ? kFp4RowBytes : kRec;   // index-list unit: bytes per record
    constexpr int KS = D / 32;                      // Q.K^T MFMA steps (32 dims each)
    constexpr int ROWB = D * 2;                     // bytes of a bf16 row in HBM
    // raw masked scores with the scale in the exponent (576-wide bf16 pages, positive scales);
    // otherwise the scores are scaled before masking, which takes any scale
    constexpr bool RAWMAX = !GATHER && D == kDqk;
    using C = Cfg<GATHER, SPARSE, D>;
    constexpr int PF = kPF;
    constexpr int VPF = kVPF;
    constexpr int DEPTH = C::DEPTH;
    constexpr int AHEAD = C::AHEAD;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    static_assert(C::LDS >= kWaves * 16 * kOutPitch, "output staging must fit in LDS");
    char* ring = smem;
    int* lidx = reinterpret_cast<int*>(smem + C::RING);
    int* lpages = reinterpret_cast<int*>(smem + C::RING + C::IDX);
    uint2* px = reinterpret_cast<uint2*>(smem + C::RING + C::IDX + C::PAGES);
    int* votes = reinterpret_cast<int*>(smem + C::RING + C::IDX + C::PAGES + C::PX);
    float* red = reinterpret_cast<float*>(px);      // end-of-pass exchanges (P no longer read)

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rb = wave & 3;           // row block
    const int h = wave >> 2;           // token half of Q.K^T, value half of P.V
    const int partner = wave ^ 4;
    const int g4 = lane >> 4, l16 = lane & 15;

    // ---- work item -> (part or sparse split, row group); row groups of one item share an XCD
    const int R = ceil_div(a.M, kRowsWg);
    const int n_items = SPARSE ? a.batch * a.num_parts : a.num_parts;
    int item, rg;
    xcd_item(blockIdx.x, n_items, R, item, rg);
    const int row = rg * kRowsWg + 16 * rb + l16;     // this lane's query row (B / C column)
    const bool row_ok = row < a.M;
    // row groups that re-read the same KV keep it in L2 (default policy); a single reader
    // streams it (nontemporal)
    auto copy = [&](const void* g, const void* l) {
        if constexpr (SHARED) dma16_shared(g, l);
        else dma16(g, l);
    };
    auto copy_s = [&](const void* sbase, unsigned voff, const void* l) {
        if constexpr (SHARED) dma16_s_shared(sbase, voff, l);
        else dma16_s(sbase, voff, l);
    };

    // ---- LDS fragment offsets that do not depend on the chunk
    // K, token tile t (tokens 16t + l16), step ks: dims 32*ks + 8*g4 (kaddr + 64*ks + 16*kRowA16*t;
    // region B for ks = 16, 17 via kaddrB + 2048*t)
    const int kaddr = l16 * kRowA16 + g4 * 16;
    int kaddrB[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) kaddrB[par] = kRegionB16 + l16 * 128 + (((4 * par + g4) ^ swzB(l16)) << 4);
    // V^T, dims 16*dt + l16 of the A operand, dt = 16h + j: lane supplies token row 4*g4 + l16/4
    // (+16 for the second half of the tokens), dims 16*dt + 8*((l16&3)>>1) + 4*(l16&1)
    const int vaddr = (4 * g4 + (l16 >> 2)) * kRowA16 + ((l16 & 3) >> 1) * 16 + (l16 & 1) * 8 + 32 * 16 * h;

    // ---- sparse gathers: load i of this lane fetches the 8 bytes at g_off of record g_tok/4 of
    // the chunk and stores them at g_dst of the ring slot: codes as 8 bf16 (16 B), the first half
    // of the scale granule as its raw first dword
    int g_tok[GATHER ? NG : 1], g_off[GATHER ? NG : 1], g_dst[GATHER ? NG : 1];
    if constexpr (FP4) {
        // lane: code granule lane & 15 (dims 32*(lane & 15) .. +31) of record lane >> 4
        const int tok = 4 * wave + (lane >> 4);
        g_tok[0] = tok * 4;
        g_off[0] = (lane & 15) * 16;
        g_dst[0] = tok * kRowA16 + (lane & 15) * 64;
    } else if constexpr (GATHER) {
#pragma unroll
        for (int i = 0; i < kGather; ++i) {
            int sl = 64 * i + lane;
            if (sl >= 8 * 37) sl -= 64;
            const int tok = 4 * wave + sl / 74;
            const int hg = sl % 74;
            const int gran = hg >> 1, half = hg & 1;
            g_tok[i] = tok * 4;
            g_off[i] = gran * 16 + half * 8;
            g_dst[i] = gran == 36 ? kChunk16 + tok * 32 + half * 16
                     : gran < 32  ? tok * kRowA16 + gran * 32 + half * 16
                                  : kRegionB16 + tok * 128 + (((2 * (gran - 32) + half) ^ swzB(tok)) << 4);
        }
    }
    // gathered records (FP4: code rows) and the FP4 scale rows, addressed with 64-bit offsets
    const char* pool = static_cast<const char*>(a.kv);
    const char* pool_sc = static_cast<const char*>(a.kv_scale);

    bf16x8 qf[KS];
    f4 acc[16];
    float m_run, l_run;
    float m_lane;     // largest score this lane has seen in the pass (for a restart's reference)

    // ---- segment start.  Q (64 rows) and, sparse, the split's index list come by direct copies
    // into LDS: Q into the ring's last two slots, which the pipeline's first chunks leave free,
    // each wave an eighth; the fragments are read from there just before the first Q.K^T.
    constexpr int QOPS = ROWB / 128;                 // 1 KB copies of Q per wave (64 rows / 8 waves)
    char* const qs = ring + (DEPTH - 2) * C::BUF;
    auto copy_q = [&](int grp) {
        const char* qg = static_cast<const char*>(a.q) + (size_t)grp * a.M * ROWB;
        // (an opaque lane id: the per-lane offsets are not hoisted out of the segment loop)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < QOPS; ++i) {
            const int j = wave + kWaves * i;
            const unsigned e = 1024 * j + 16 * ln;
            const int r = rg * kRowsWg + (int)(e / ROWB);     // rows past M read row 0
            dma16_s(qg, (unsigned)((r < a.M ? r : 0) * ROWB) + e % ROWB, qs + 1024 * j);
        }
    };
    // sparse: the split's entries [t0, t1) as raw index values, 64 per copy (entries past t1
    // read entry t0 and are marked unused later)
    auto copy_idx = [&](int grp, int t0, int t1) {
        const int nch = ceil_div(t1 - t0, kChunk);
        const int* ig = a.indices + (size_t)grp * a.topk + t0;
#pragma unroll
        for (int i = 0; i < kMaxSparseSplit / (64 * kWaves); ++i) {
            const int j = wave + kWaves * i;
            if (64 * j < nch * kChunk) {
                const int e = 64 * j + lane;
                dma4(ig + (e < t1 - t0 ? e : 0), lidx + 64 * j);
            }
        }
    };
    // Q fragments (B operand of S^T): dims 32*ks + 8*g4 .. +7 of this lane's row, from the copy
    // (every wave's copies have landed: the caller waited for this wave's, a barrier for the rest)
    auto read_q = [&]() {
        const char* qrow = qs + (16 * rb + l16) * ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 v = *reinterpret_cast<const uint4*>(qrow + (ks * 32 + g4 * 8) * 2);
            if (!row_ok) v = make_uint4(0, 0, 0, 0);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
    };

    // win0 (paged): lane i holds the block-table entry of page t0/64 + i
    auto run_segment = [&](int grp, int t0, int t1, int L, bool final_out, int slot, int win0) {
        const int nch = ceil_div(t1 - t0, kChunk);
        m_run = -INFINITY;
        const int limit = a.causal ? (L - a.s_q + row / a.h_q) : (L - 1);

        // sparse: the copied index values become record numbers in place (-1 for unused entries
        // and up to the end of the last chunk)
        if constexpr (SPARSE) {
            __syncthreads();                 // every wave's index copies have landed
            constexpr int kPer = kMaxSparseSplit / (kWaves * 64);
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int e = threadIdx.x + j * kWaves * 64;
                if (e < nch * kChunk) {
                    const int v = lidx[e];
                    lidx[e] = (e < t1 - t0 && v >= 0 && v < a.kv_rows) ? v : -1;
                }
            }
            __syncthreads();
        }

        // paged: page numbers of the segment, 64 at a time into a per-wave LDS window (a lookup
        // then never waits on the vector-memory counter, which also counts the KV copies); the
        // first window from the caller
        int bt_base = 0;
        if constexpr (!SPARSE) lpages[wave * 64 + lane] = win0;
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

        // ---- paged copies of one chunk, spread over the waves and over the MFMAs.  Chunks past
        // the segment's end re-copy its last chunk into their (unused) slot, which keeps the number
        // of copies per chunk fixed.
        struct Plan {
            const char* base;                      // first row of the chunk in HBM
            char* dst;
            int nrows;
        };
        auto plan_for = [&](int c) {
            Plan p;
            const int cc = min(c, nch - 1);
            p.dst = ring + (c % DEPTH) * C::BUF;
            const int tb = t0 + cc * kChunk;
            p.nrows = min(kChunk, t1 - tb);
            p.base = nullptr;
            if constexpr (!GATHER) {
                const int page = page_of(cc >> 1);
                p.base = static_cast<const char*>(a.kv) + ((size_t)page * kPage + (tb & 63)) * ROWB;
            }
            return p;
        };
        auto copy_op = [&](const Plan& p, int j) {
            const int q = wave + kWaves * j;
            if (j < kChunk / kWaves) {   // region A rows
                const int rr = min(q, p.nrows - 1);
                copy_s(p.base + rr * ROWB, (unsigned)lane << 4, p.dst + q * kRowA16);
            } else {                     // region B: 8 rows of 128 B per copy (parts 0..3, repeated)
                const int part = (q - kChunk) & 3;
                const int sl = part * 64 + lane;
                const int br = sl >> 3;
                const int rr = min(br, p.nrows - 1);
                copy(p.base + rr * ROWB + (64 + ((sl & 7) ^ swzB(br))) * 16,
                     p.dst + kRegionB16 + part * 1024);
            }
        };

        // ---- sparse: load i of chunk c into registers; conversion of those registers into chunk
        // c's ring slot.  Chunks past the segment's end gather its last chunk again (unused slot).
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        using GV = std::conditional_t<FP4, u32x4, u32x2>;
        GV gv[GATHER ? NG : 1];
        int g_rec[GATHER ? NG : 1];       // record of load i, -1: none (reads record 0)
        unsigned short g_sc = 0;      // FP4: the two scale bytes of this lane's 32 values
        // paged gathers of the current chunk (wave-uniform): record of its first token, and how
        // many of its tokens are read (0 for a page outside the cache)
        unsigned gp_rec0 = 0;
        int gp_n = 0;
        auto gather = [&](int c, int i) {
            const int cc = min(c, nch - 1);
            int rec;
            if constexpr (SPARSE) {
                rec = *reinterpret_cast<const int*>(reinterpret_cast<const char*>(lidx) + cc * kChunk * 4 + g_tok[i]);
            } else {
                // paged records: a chunk lies inside one page (segments start on a page); tokens
                // past the segment's end read nothing.  Gather 0 of a chunk comes first.
                if (i == 0) {
                    const int tb = t0 + cc * kChunk;
                    const int pg = page_of(cc >> 1);
                    const bool pg_ok = pg >= 0 && (long long)pg * kPage < a.kv_rows;
                    gp_rec0 = (unsigned)pg * kPage + (tb & 63);
                    gp_n = pg_ok ? min(kChunk, t1 - tb) : 0;
                }
                const int lt = g_tok[i] >> 2;
                rec = lt < gp_n ? (int)(gp_rec0 + lt) : -1;
            }
            g_rec[i] = rec;
            const size_t rr = rec >= 0 ? (size_t)rec : 0;
            const GV* gp = reinterpret_cast<const GV*>(pool + rr * REC + g_off[i]);
            if constexpr (SHARED) gv[i] = *gp;
            else gv[i] = __builtin_nontemporal_load(gp);
            if constexpr (FP4)
                g_sc = *reinterpret_cast<const unsigned short*>(pool_sc + rr * (kFp4RowBytes >> kFp4ScaleShift) +
                                                                (g_off[i] >> 3));
        };
        // FP4: quarter w (8 values, dims 32*(lane & 15) + 8w .. +7) of this lane's registers into
        // chunk c's ring slot.  Code bytes 0..7 belong to block 2*(lane & 15), bytes 8..15 to the
        // next block.
        auto convert_fp4 = [&](int c, int w) {
            char* slot = ring + (c % DEPTH) * C::BUF;
            // an unused token converts to zeros (record 0's bytes, which it read, are not its own)
            const bool none = g_rec[0] < 0;
            const unsigned codes = none ? 0u : gv[0][w];
            const float sc = none ? 0.f : __builtin_amdgcn_cvt_f32_fp8((int)((unsigned)g_sc >> (8 * (w >> 1))), 0);
            unsigned o[4];
            // with a unit scale the conversion is exact; the block scale multiplies in fp32,
            // exactly, and the product is a bf16 value
#define MLA_FP4_PAIR(B_)                                                              \
    {                                                                                 \
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, B_);     \
        o[B_] = pack_bf16x2(v[0] * sc, v[1] * sc);                                    \
    }
            MLA_FP4_PAIR(0) MLA_FP4_PAIR(1) MLA_FP4_PAIR(2) MLA_FP4_PAIR(3)
#undef MLA_FP4_PAIR
            *reinterpret_cast<uint4*>(slot + g_dst[0] + 16 * w) = make_uint4(o[0], o[1], o[2], o[3]);
            // token validity: 1 for a record, NaN for an unused entry (masked off)
            if (w == 0 && (lane & 15) == 0)
                *reinterpret_cast<unsigned*>(slot + kChunk16 + (g_tok[0] >> 2) * 32) =
                    g_rec[0] < 0 ? 0x7fc00000u : 0x3f800000u;
        };
        auto convert = [&](int c, int i) {
            char* slot = ring + (c % DEPTH) * C::BUF;
            // an unused entry converts to zeros (record 0's bytes, which it read, are not its own)
            const GV r = g_rec[i] < 0 ? GV{} : gv[i];
            uint4 lo = __builtin_bit_cast(uint4, fp8x8_to_bf16(r.x, r.y));
            // scale granule: the raw fp32 scale, NaN for an unused entry (masked off)
            const unsigned sc = g_rec[i] < 0 ? 0x7fc00000u : r.x;
            lo.x = g_off[i] == 36 * 16 ? sc : lo.x;
            *reinterpret_cast<uint4*>(slot + g_dst[i]) = lo;
        };

        // ---- LDS fragments
        auto kfrag = [&](const char* buf, int t, int ks) -> bf16x8 {
            const int off = ks < 16 ? kaddr + 64 * ks + 16 * kRowA16 * t : kaddrB[ks & 1] + 16 * 128 * t;
            return *reinterpret_cast<const bf16x8*>(buf + off);
        };
        auto vfrag = [&](const char* buf, int j) -> bf16x8 {
            const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr + 32 * j));
            const short4v v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(buf + vaddr + 32 * j + 16 * kRowA16));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
        };

        // S^T of chunk c, tile t x this wave's 16 rows: two MFMA chains s2[ks&1] (the other wave
        // of the SIMD fills the MFMA latency).  side(ks) runs between the steps.
        auto qk = [&](int c, int t, f4 (&s2)[2], auto&& side) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            s2[0] = s2[1] = f4{0.f, 0.f, 0.f, 0.f};
            bf16x8 kf[PF];
#pragma unroll
            for (int i = 0; i < PF - 1; ++i) kf[i] = kfrag(buf, t, i);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + PF - 1 < KS) kf[(ks + PF - 1) % PF] = kfrag(buf, t, ks + PF - 1);
                s2[ks & 1] = mfma16(kf[ks % PF], qf[ks], s2[ks & 1]);
                side(ks);
            }
        };
        // O^T[256h + 16j .. +15][rows] += V^T P^T over chunk c's 32 tokens, j = 0..15; side(j)
        auto pv = [&](int c, bf16x8 pT, auto&& side) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            bf16x8 vf[VPF];
#pragma unroll
            for (int i = 0; i < VPF - 1; ++i) vf[i] = vfrag(buf, i);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j + VPF - 1 < 16) vf[(j + VPF - 1) % VPF] = vfrag(buf, j + VPF - 1);
                acc[j] = mfma16(vf[j % VPF], pT, acc[j]);
                side(j);
            }
        };

        // ---- masking of tile t of chunk c: masked scores in log2 units (paged: raw, scaled
        // later; sparse: scaled), the tile's largest scaled score, and token scales
        struct Tile {
            f4 s;
            float mx;       // largest scaled score of the tile in this lane
            float tsc[4];   // sparse: token scales (0 for masked tokens)
        };
        auto mask_tile = [&](int c, int t, f4 s, Tile& T) {
            const char* buf = ring + (c % DEPTH) * C::BUF;
            const int tb = t0 + c * kChunk;
            if constexpr (RAWMAX) {
                // raw scores; a positive scale commutes with the maximum and is applied in the
                // exponent (the launcher sends other scales to another kernel)
                const int bnd = min(t1, limit + 1) - tb - 16 * t - 4 * g4;    // valid: i < bnd
#pragma unroll
                for (int i = 0; i < 4; ++i) T.s[i] = i < bnd ? s[i] : -INFINITY;
                T.mx = fmaxf(fmaxf(T.s[0], T.s[1]), fmaxf(T.s[2], T.s[3])) * a.scale_log2;
            } else if constexpr (!GATHER) {
                // scaled scores (log2 units), masked
                const int bnd = min(t1, limit + 1) - tb - 16 * t - 4 * g4;
#pragma unroll
                for (int i = 0; i < 4; ++i) T.s[i] = i < bnd ? s[i] * a.scale_log2 : -INFINITY;
                T.mx = fmaxf(fmaxf(T.s[0], T.s[1]), fmaxf(T.s[2], T.s[3]));
            } else {
                // fp8 pages also apply the row's causal limit: token i of the lane is visible
                // while i <= lim
                const int lim = SPARSE ? 3 : limit - tb - 16 * t - 4 * g4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * t + 4 * g4 + i;
                    // NaN marks an unused entry or a position past the list
                    const float sc = *reinterpret_cast<const float*>(buf + kChunk16 + tok * 32);
                    const bool valid = (sc == sc) & (i <= lim);
                    if constexpr (FP4) {
                        T.s[i] = valid ? s[i] * a.scale_log2 : -INFINITY;
                    } else {
                        T.tsc[i] = valid ? sc : 0.f;
                        T.s[i] = valid ? s[i] * (a.scale_log2 * sc) : -INFINITY;
                    }
                }
                T.mx = fmaxf(fmaxf(T.s[0], T.s[1]), fmaxf(T.s[2], T.s[3]));
            }
        };
        // probabilities of the own tile under the row's reference: 4 bf16 in two dwords
        auto probs = [&](const Tile& T) -> uint2 {
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (!RAWMAX) p[i] = exp2_fast(T.s[i] - m_use);
                else p[i] = exp2_fast(__builtin_fmaf(T.s[i], a.scale_log2, -m_use));
                l_run += p[i];
                if constexpr (GATHER && !FP4) p[i] *= T.tsc[i];
            }
            return make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
        };
        // B operand element j of lane (l16, g4) is token (j < 4 ? 4*g4 + j : 16 + 4*g4 + j - 4):
        // tile 0's then tile 1's probabilities of this lane's row
        auto p_operand = [&](uint2 own, uint2 other) {
            const uint4 v = h == 0 ? make_uint4(own.x, own.y, other.x, other.y)
                                   : make_uint4(other.x, other.y, own.x, own.y);
            return __builtin_bit_cast(bf16x8, v);
        };
        // after the barrier that follows the vote of chunk c: any vote in the workgroup?
        auto any_vote = [&](int c) {
            int any = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) any |= votes[(c & 1) * kWaves + w];
            return __builtin_amdgcn_readfirstlane(any) != 0;
        };
        auto no_side = [](int) {};
        // gathered chunks, during the Q.K^T steps of a chunk: conversion of chunk cn's registers,
        // then the loads of chunk cn+1 into them (FP4: four conversion quarters, then the load)
        auto gather_side = [&](int cn, int ks) {
            if constexpr (FP4) {
                if ((ks & 1) == 1 && ks < 8) convert_fp4(cn, ks >> 1);
                if (ks == 8) gather(cn + 1, 0);
            } else if ((ks & 1) == 0 && ks / 2 < NG) {
                convert(cn, ks / 2);
                gather(cn + 1, ks / 2);
            }
        };
        // copies are counted exactly (AHEAD-1 later chunks may still be in flight)
        auto wait_chunk = [&]() {
            if constexpr (AHEAD - 1 == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((AHEAD - 1) * C::OPS) : "memory");
        };

        // ---- passes over the segment (a second one only after a restart vote).  A vote does not
        // leave the chunk loop early: the pass runs to its end (its results are discarded), so
        // the loop has a single exit and m_lane sees every score of the segment.
        for (int pass = 0;; ++pass) {
            l_run = 0.f;
            m_lane = -INFINITY;
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
            bool restart = false;
            uint2 p_own;
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
                if constexpr (FP4) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) convert_fp4(0, w);
                } else {
#pragma unroll
                    for (int i = 0; i < NG; ++i) convert(0, i);
                }
#pragma unroll
                for (int i = 0; i < NG; ++i) gather(1, i);
            }
            // chunk 0: Q.K^T of both tiles (the row's reference needs all 32 tokens; the copies of
            // chunk AHEAD, or the conversion of chunk 1 and the gathers of chunk 2, spread over
            // it), reference, probabilities of the own tile
            __syncthreads();
            if (pass == 0) {
                // Q from its copy; every wave has read it before the slots are refilled
                read_q();
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __syncthreads();
            }
            {
                const Plan p = plan_for(AHEAD);
                auto side0 = [&](int ks) {
                    if constexpr (!GATHER) {
                        if ((ks & 1) == 0 && ks / 2 < C::OPS) copy_op(p, ks / 2);
                    } else {
                        gather_side(1, ks);
                    }
                };
                f4 s0[2], s1[2];
                qk(0, 0, s0, side0);
                qk(0, 1, s1, no_side);
                Tile T0, T1;
                mask_tile(0, 0, s0[0] + s0[1], T0);
                mask_tile(0, 1, s1[0] + s1[1], T1);
                float mx = fmaxf(T0.mx, T1.mx);
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                m_lane = fmaxf(m_lane, mx);
                if (m_run == -INFINITY) m_run = mx;     // a restart pass keeps its reference
                p_own = probs(h == 0 ? T0 : T1);
                px[(0 * kWaves + wave) * 64 + lane] = p_own;
                if (lane == 0) votes[wave] = 0;
            }
            for (int k = 1; k < nch; ++k) {
                if constexpr (!GATHER) wait_chunk();
                // chunk k in LDS; probabilities and votes of chunk k-1 visible; slot (k-2) % DEPTH free
                __syncthreads();
                restart = restart | any_vote(k - 1);
                const uint2 p_other = px[(((k - 1) & 1) * kWaves + partner) * 64 + lane];
                const Plan p = plan_for(k + AHEAD);
                f4 s2[2];
                // S^T(k) of the own tile on the MFMAs while chunk k+AHEAD is copied (sparse:
                // chunk k+1 is converted and chunk k+2 gathered)
                qk(k, h, s2, [&](int ks) {
                    if constexpr (!GATHER) {
                        if ((ks & 1) == 0 && ks / 2 < C::OPS) copy_op(p, ks / 2);
                    } else {
                        gather_side(k + 1, ks);
                    }
                });
                // O^T += V^T P^T (k-1) on the MFMAs while S^T(k) is masked and turned into
                // probabilities
                Tile T;
                bool outgrown = false;
                uint2 p_next;
                pv(k - 1, p_operand(p_own, p_other), [&](int j) {
                    if (j == 3) {
                        mask_tile(k, h, s2[0] + s2[1], T);
                        m_lane = fmaxf(m_lane, T.mx);
                        // also true for a finite score in a row without a reference
                        outgrown = T.mx > m_run + kRefSlack;
                    }
                    if (j == 7) p_next = probs(T);
                });
                p_own = p_next;
                px[((k & 1) * kWaves + wave) * 64 + lane] = p_own;
                const bool v = __builtin_amdgcn_ballot_w64(outgrown) != 0;
                if (lane == 0) votes[(k & 1) * kWaves + wave] = v ? 1 : 0;
            }
            __syncthreads();                   // votes and probabilities of the last chunk visible
            restart = restart | any_vote(nch - 1);
            if (!restart) {
                const uint2 p_other = px[(((nch - 1) & 1) * kWaves + partner) * 64 + lane];
                pv(nch - 1, p_operand(p_own, p_other), no_side);
            }
            // the copies past the segment's end land first
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // (the second pass, whose reference is the segment maximum, cannot vote; the bound on
            // the passes is a guard)
            if (!restart || pass == 1) break;
            // run the pass again with each row's maximum over the segment (both tiles) as reference
            float mx = m_lane;
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            __syncthreads();                   // exchanged probabilities no longer read
            red[wave * 64 + lane] = mx;
            __syncthreads();
            m_run = fmaxf(mx, red[partner * 64 + lane]);
            __syncthreads();
        }

        // ---- row sums: the four lanes of a row, then the partner wave's tile
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        __syncthreads();                    // exchanged probabilities no longer read
        red[wave * 64 + lane] = l_run;
        __syncthreads();
        l_run += red[partner * 64 + lane];
        float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
        if (final_out && a.sinks) {
            // the head's attention sink joins the denominator (a split row gets it in the combine)
            const float sk = a.sinks[(row_ok ? row : 0) % a.h_q];
            const float hi = fmaxf(lse_v, sk), lo = fminf(lse_v, sk);
            const float tot = lo == -INFINITY ? hi : hi + log1pf(expf(lo - hi));
            inv *= l_run > 0.f ? expf(lse_v - tot) : 0.f;
            lse_v = tot;
        }
        if (row_ok && g4 == 0 && h == 0) {
            if (final_out) a.lse[(size_t)grp * a.M + row] = lse_v;
            else a.part_lse[(size_t)slot * a.M + row] = lse_v;
        }
        // ---- output through LDS, so that every store instruction writes whole 128-byte lines:
        // the wave's 16 rows x 256 values go to its own LDS area (rows padded by 16 B), then out
        // again as 16 contiguous bytes per lane
        __syncthreads();                    // the exchange area is read: all of LDS is free
        char* stg = smem + wave * (16 * kOutPitch);
        const int row0 = rg * kRowsWg + 16 * rb;
        // computed here, not hoisted out of the segment and pass loops, where they would hold
        // registers through the chunk loop
        int ln = lane, nrow = a.M - row0;
        asm volatile("" : "+v"(ln), "+s"(nrow));
        if (final_out) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const f4 v = acc[j] * inv;
                *reinterpret_cast<uint2*>(stg + l16 * kOutPitch + j * 32 + g4 * 8) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
            char* obase = static_cast<char*>(a.out) + ((size_t)grp * a.M + row0) * (kDv * 2) + 512 * h;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 2 * i + (ln >> 5), cgr = ln & 31;
                const uint4 v = *reinterpret_cast<const uint4*>(stg + r * kOutPitch + cgr * 16);
                if (r < nrow) *reinterpret_cast<uint4*>(obase + (size_t)r * (kDv * 2) + cgr * 16) = v;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                *reinterpret_cast<f4*>(stg + l16 * kOutPitch + j * 64 + g4 * 16) = acc[j] * inv;
            char* pbase = reinterpret_cast<char*>(a.part_o) + ((size_t)slot * a.M + row0) * (kDv * 4) + 1024 * h;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint4 v = *reinterpret_cast<const uint4*>(stg + r * kOutPitch + ln * 16);
                if (r < nrow) *reinterpret_cast<uint4*>(pbase + (size_t)r * (kDv * 4) + ln * 16) = v;
            }
        }
        __syncthreads();                    // LDS (ring, index list, exchanges) free for the next segment
    };

    if constexpr (!SPARSE) {
        const int* meta = a.tile_meta + (size_t)item * kMetaInts;
        const int b0 = meta[0], blk0 = meta[1], b1 = meta[2], blk1 = meta[3], slot0 = meta[4];
        for (int bb = b0; bb <= b1 && bb < a.batch; ++bb) {
            // A segment's first loads go out together, one memory round trip before its first KV
            // copy: the copy of Q, the first 64 block-table entries from page lo (in bounds of
            // the row; entries past the sequence are never used), its length and split count.
            // All are waited for (the empty asm reads the window) before the KV copies start, so
            // no load the compiler tracks is pending behind a copy.  (The copy of Q goes first:
            // the compiler's waits on the later loads then cover it.)
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
    } else {
        const int grp = item / a.num_parts;
        const int split = item % a.num_parts;
        const int e0 = split * a.split_len;
        const int e1 = min(e0 + a.split_len, a.topk);
        if (e0 < e1) {
            // the index list first, then Q: the first gathers wait only for the list
            copy_idx(grp, e0, e1);
            copy_q(grp);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(QOPS) : "memory");
            run_segment(grp, e0, e1, 0, a.num_parts == 1, grp * a.num_parts + split, 0);
        }
    }
}

}  // namespace rows

hipError_t launch_decode_rows(const AttnArgs& a, bool sparse, hipStream_t stream) {
    const int items = sparse ? a.batch * a.num_parts : a.num_parts;
    const int R = (a.M + rows::kRowsWg - 1) / rows::kRowsWg;
    const dim3 grid(items * R), block(rows::kWaves * 64);
#define MLA_ROWS_LAUNCH(MODE_, D_)                                                                                 \
    if (R > 1) hipLaunchKernelGGL((rows::mla_decode_rows_kernel<MODE_, true, D_>), grid, block, 0, stream, a);  \
    else hipLaunchKernelGGL((rows::mla_decode_rows_kernel<MODE_, false, D_>), grid, block, 0, stream, a);
    if (sparse) {
        MLA_ROWS_LAUNCH(rows::kSparseFp8, kDqk)
    } else if (a.kv_fp4) {
        MLA_ROWS_LAUNCH(rows::kPagedFp4, kDv)
    } else if (a.kv_fp8) {
        MLA_ROWS_LAUNCH(rows::kPagedFp8, kDqk)
    } else if (a.d_qk == kDv) {
        MLA_ROWS_LAUNCH(rows::kPagedBf16, kDv)
    } else {
        MLA_ROWS_LAUNCH(rows::kPagedBf16, kDqk)
    }
#undef MLA_ROWS_LAUNCH
    return hipGetLastError();
}

}  // namespace mla
