// The allocation-free paged decode entry point: mla_decode_paged with its split-KV workspace in
// a fixed-size array that the library holds on each GPU, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
#include "mla.h"
#include "mla_internal.h"

#include <mutex>

// The workspace of mla_decode_paged_noalloc.  The code object's load places one copy on every GPU
// the library runs on, each at its own address, held until the process ends.  In host code the
// name below only stands in for the symbol: kernels and copies get the device address that
// hipGetSymbolAddress returns for the current device, never the name itself.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// Address of the current device's copy of `scratch`, looked up on the first call on that device
// with it current.
mla_status_t scratch_of_current_device(size_t need, void** ptr, size_t* bytes) {
    if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
    return MLA_OK;
}

}  // namespace

extern "C" mla_status_t mla_decode_paged_noalloc(const void* q, const void* kcache, int64_t num_blocks,
                                                 const int32_t* block_table, int max_blocks,
                                                 const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                                                 float softmax_scale, int causal,
                                                 const int32_t* tile_meta, const int32_t* num_splits,
                                                 int num_parts, void* out, float* lse, void* stream) {
    return mla::decode_paged_scratch(q, kcache, num_blocks, block_table, max_blocks, cache_seqlens, batch, s_q,
                                     h_q, softmax_scale, causal, tile_meta, num_splits, num_parts, out, lse,
                                     stream, scratch_of_current_device);
}
