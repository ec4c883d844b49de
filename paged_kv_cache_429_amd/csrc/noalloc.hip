// paged_attn_decode_noalloc: the decode with its scratch in a fixed device
// array instead of a caller workspace, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops).
//
// The decode's scratch (arrival words, split partials, the prefix pass's
// per-tile runs) lives in `scratch`, a file-scope device array that each
// device holds for the life of the process. Its device address is taken once
// per device with hipGetSymbolAddress (the array's name in host code is only
// a stand-in, never a device address) and kept; the kernels get that address
// as their workspace argument. The arrival words are tagged with each call's
// epoch, so nothing in the array has to start at zero. Calls that overlap on
// one device share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/paged_attn.h"

static constexpr size_t kScratchBytes = (size_t)PA_DECODE_NOALLOC_SCRATCH_BYTES;

// The decode scratch of paged_attn_decode_noalloc (one copy per device).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of `scratch` on the current device (nullptr on failure),
// taken the first time this device asks.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    return g_ptr[dev];
}

}  // namespace

extern "C" int paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                         const uint16_t* k_scales, const uint16_t* v_scales,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* context_lens, int max_context_len, int num_seqs,
                                         int num_blocks, int block_size, int n_heads, int n_kv_heads, int d_head,
                                         int dtype, int kv_bits, void* out, int partition_blocks, void* stream) {
    const size_t need = paged_attn_decode_workspace_size(num_seqs, n_heads, n_kv_heads, d_head,
                                                         max_context_len > 0 ? max_context_len : 1,
                                                         partition_blocks);
    if (need > kScratchBytes) return PA_ERR_SCRATCH;
    void* ws = scratch_ptr();
    if (!ws) return PA_ERR_HIP;
    return paged_attn_decode(q, k_pool, v_pool, k_scales, v_scales, block_tables, max_blocks_per_seq, context_lens,
                             max_context_len, num_seqs, num_blocks, block_size, n_heads, n_kv_heads, d_head, dtype,
                             kv_bits, out, ws, kScratchBytes, partition_blocks, stream);
}
