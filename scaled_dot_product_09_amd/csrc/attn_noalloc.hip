// attn_noalloc.hip — the split-key forward for callers that cannot allocate.
//
// attn_fwd_split needs a caller workspace for the key ranges' fp32 partial
// results. Callers that cannot call hipMalloc (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation) use
// attn_fwd_split_noalloc instead: the partial results go to a file-scope
// device array, `scratch`, of ATTN_NOALLOC_SCRATCH_BYTES, which every GPU the
// library runs on holds from the library's first use on it until the
// process ends. The kernels are attn_fwd_split's own.
//
// The array's address on a device comes from hipGetSymbolAddress, taken
// once per device with that device current (each GPU holds its own copy at
// its own address); host code passes only that address to the kernels,
// never the array's name (a host-side stand-in). Every call on a GPU shares
// that GPU's array: calls that overlap in time on one GPU (different
// streams) race on it. Nothing in it needs clearing: every partial result
// is written by exactly one workgroup before the combine kernel reads it.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/attn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of this device's scratch array (nullptr on failure).
void* scratch_on_current_device() {
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

extern "C" int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* out,
                                      int B, int Hq, int Hkv, int Sq, int Skv, int D,
                                      float scale, int causal, int dtype, int n_split, hipStream_t stream) {
    // Size first (host arithmetic only): attn_split_workspace returns 0 for
    // shapes that need no workspace or are invalid (attn_fwd_split then
    // reports the shape error).
    const size_t need = attn_split_workspace(B, Hq, Sq, D, n_split);
    if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_on_current_device();
        if (!ws) return ATTN_ERR_HIP;
    }
    return attn_fwd_split(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, n_split, ws,
                          (size_t)ATTN_NOALLOC_SCRATCH_BYTES, stream);
}
