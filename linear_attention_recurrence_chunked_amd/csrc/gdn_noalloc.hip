// gdn_noalloc.hip -- gdn_prefill_noalloc: the chunked prefill with its workspace in a fixed
// device array of the library, for callers that cannot allocate device memory.
//
// The array is a file-scope device variable (one copy per GPU, held from the library's load
// until the process ends).  In host code its name is only a stand-in symbol, so the device
// address of each GPU's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; every launch takes that address.  Nothing here calls an
// allocator: the work is gdn_prefill_ex's, with this array as its workspace.
//
// Every call on one GPU uses that GPU's single array, so calls that overlap in time on one
// GPU (two streams, two threads) race on it; calls on one stream are ordered and safe.  The
// prefill's kernels write every workspace byte they read within the call, so the contents a
// previous call leaves behind are never read.
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr size_t kScratchBytes = (size_t)GDN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_ptr[kMaxDevices] = {};

// Device address of the current device's copy of the array (nullptr on a HIP error).
void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace
}  // namespace gdn

extern "C" {

size_t gdn_noalloc_scratch_bytes(void) { return gdn::kScratchBytes; }

gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *alpha,
                               const float *beta, const float *initial_state,
                               const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_T,
                               int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, void *y,
                               float *final_state, void *stream)
{
    // the size check is a pure function of the arguments: nothing reaches HIP before it
    if (num_seqs <= 0 || total_T < 0 || H <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128)) return GDN_ERR_UNSUPPORTED;
    const size_t need = gdn_prefill_workspace_bytes(num_seqs, total_T, H, d_k, d_v, dtype);
    if (need > gdn::kScratchBytes) return GDN_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    if (need > 0) {
        ws = gdn::scratch_address();
        if (!ws) return GDN_ERR_HIP;
    }
    return gdn_prefill_ex(q, k, v, alpha, beta, initial_state, cu_seqlens, num_seqs, total_T,
                          H, d_k, d_v, dtype, y, final_state, ws, need, stream, 0, 0);
}

}  // extern "C"
