// Device helpers shared by the gfx950 decode kernels: operand types, the LDS chunk layout,
// MFMA and conversion wrappers, and the HBM -> LDS copy.
#pragma once

#include "mla_internal.h"

#include <cmath>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

constexpr int kRowBytes = kDqk * 2;       // 1152: one bf16 row in HBM
constexpr int kChunkBytes = kChunk * kRowBytes;
// LDS chunk layout: region A holds dims 0..511 of the 32 rows (1024 B per row), region B the
// 64 RoPE dims (128 B per row), so each region can be filled by whole-wave 1 KB writes.
constexpr int kRowA = 1024;
constexpr int kRegionB = kChunk * kRowA;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online softmax with a lagging reference: probabilities are exp2(x - m) with m the row's
// reference, which only moves when the row maximum exceeds it by more than kSlack, so
// p <= 2^kSlack and the accumulator is rescaled rarely.  The final O = acc / l and
// LSE = m + log2(l) use the same reference, so the result is exact up to rounding.
constexpr float kSlack = 8.f;

// --------------------------------------------------------------------------
// Small helpers
// --------------------------------------------------------------------------
__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// LDS row layout: row r holds 72 granules of 16 B (8 dims each); granule c sits at slot
// c ^ swz(r).  swz permutes within aligned groups of 8 granules so that (a) 8 consecutive
// rows reading the same granule (QK^T A operand, ds_read_b128) hit 8 distinct 16-B bank
// groups and (b) 4 consecutive rows reading the same 32-B pair (V^T transposed read) hit 4
// distinct 32-B bank groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
// granule c (0..63) of row r in region A; granule c (0..7) of row r in region B
__device__ __forceinline__ int lds_a(int r, int c) { return r * kRowA + ((c ^ swz(r)) << 4); }
__device__ __forceinline__ int lds_b(int r, int c) { return kRegionB + r * 128 + ((c ^ swz(r)) << 4); }

// Work item and row group of workgroup `bid` when each of n_items work items takes R workgroups.
// Workgroups go to the 8 XCDs round robin by block index: the R row groups of each of the first
// n_items & ~7 items land on one XCD, back to back, so that the later readers of a KV chunk hit
// that XCD's L2; the items beyond those take the remaining workgroups in order.
__device__ __forceinline__ void xcd_item(int bid, int n_items, int R, int& item, int& rg) {
    const int full = n_items & ~7;
    if (bid < full * R) {
        const int xcd = bid & 7, k = bid >> 3;
        item = (k / R) * 8 + xcd;
        rg = k % R;
    } else {
        const int t = bid - full * R;
        item = full + t / R;
        rg = t % R;
    }
}

__device__ __forceinline__ f4 mfma16(bf16x8 a, bf16x8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane L's 16 bytes land at
// LDS byte lds_addr + 16*L.  Written as a statement the compiler does not see as an LDS
// store, so it does not stall reads of the other LDS buffer on this copy; the caller waits
// with s_waitcnt vmcnt before reading the destination.  No register is written.  The KV
// cache is streamed once per call, so the copy is nontemporal (nt): measured on MI355X it
// lifts a random-page 604 MB stream from about 5.8 to 6.9 TB/s.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_ptr) {
    const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_ptr;
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
}

// The same copy with the default cache policy: for KV that several workgroups (the row groups
// of one sequence, launched back to back on one XCD) read, so later readers hit in L2.
__device__ __forceinline__ void dma16_shared(const void* gptr, const void* lds_ptr) {
    const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_ptr;
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
}

// The same two copies with the address split into a wave-uniform base (SGPRs) and a 32-bit
// per-lane offset, so a row copy needs no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff, const void* lds_ptr) {
    const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_ptr;
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma16_s_shared(const void* sbase, unsigned voff, const void* lds_ptr) {
    const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_ptr;
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}

// 4-byte copy of each lane's global address into LDS (lane i writes at m0 + 4 * i).
__device__ __forceinline__ void dma4(const void* gptr, const void* lds_ptr) {
    const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_ptr;
    asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
}

// Nontemporal 16-byte load of streamed KV data into registers.
__device__ __forceinline__ uint4 load_nt(const void* p) {
    typedef unsigned u4v __attribute__((ext_vector_type(4)));
    const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, v);
}

// 8 e4m3 codes (two dwords) -> 8 bf16, exact
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(unsigned lo, unsigned hi) {
#define MLA_CVT(w, h) __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, h))
    const uint4 v = make_uint4(MLA_CVT(lo, false), MLA_CVT(lo, true), MLA_CVT(hi, false), MLA_CVT(hi, true));
#undef MLA_CVT
    return __builtin_bit_cast(bf16x8, v);
}

// fp8 record rows in LDS (640 B = 40 granules of 16 B): granule g of row r sits at slot
// g ^ swz8(r), an XOR on the low three granule bits that keeps the 16 rows of a K fragment read
// (ds_read_b64) and of a V^T transposing read (ds_read_b64_tr_b8) on distinct banks (measured)
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ (((r >> 4) & 1) << 2); }

// 16 e4m3 codes -> 16 bf16 (exact: every finite e4m3 value is a bf16 value)
__device__ __forceinline__ void fp8x16_to_bf16(uint4 c, uint4& lo, uint4& hi) {
#define MLA_CVT(w, h) __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, h))
    lo = make_uint4(MLA_CVT(c.x, false), MLA_CVT(c.x, true), MLA_CVT(c.y, false), MLA_CVT(c.y, true));
    hi = make_uint4(MLA_CVT(c.z, false), MLA_CVT(c.z, true), MLA_CVT(c.w, false), MLA_CVT(c.w, true));
#undef MLA_CVT
}

}  // namespace mla
