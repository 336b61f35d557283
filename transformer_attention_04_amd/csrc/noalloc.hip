// sdpa_fwd_noalloc: sdpa_fwd without a caller workspace, for callers that
// cannot allocate device memory while they run (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  The only forward
// path that needs scratch memory is the split-KV decode (its per-split partial
// outputs and logsumexps, merged by a second kernel); here they go to a
// file-scope device array, `scratch`, of kNoallocScratchBytes per device.
//
// The array's device address is looked up once per device with
// hipGetSymbolAddress (the host-side name of a __device__ array is not a
// device address), on the entry point's first call on that device, and kept;
// every later call uses that pointer.  Nothing is allocated and nothing needs
// clearing: the split kernel writes every partial the merge reads, empty
// splits included.  All calls on one device share its array, so calls that
// overlap on one device (on different streams, or from several threads) race.
#include "sdpa.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"

namespace {

constexpr size_t kNoallocScratchBytes = SDPA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
std::mutex g_scratch_mu;

}  // namespace

extern "C" sdpa_status sdpa_fwd_noalloc(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* k,
                                        const sdpa_tensor4* v, const sdpa_tensor4* attn_mask, sdpa_dtype mask_dtype,
                                        double dropout_p, int is_causal, const double* scale, int enable_gqa,
                                        const sdpa_tensor4* out, const sdpa_tensor4* lse, int num_splits,
                                        void* stream) {
    size_t need = 0;
    sdpa_status st = sdpa_fwd_workspace_size(dtype, q, k, v, attn_mask, is_causal, enable_gqa, num_splits, &need);
    if (st != SDPA_OK) return st;
    if (need > kNoallocScratchBytes)
        return sdpa::record_error(SDPA_ERR_UNSUPPORTED,
                                  "this call needs %zu bytes of split-KV scratch; sdpa_fwd_noalloc holds %zu "
                                  "(pass fewer splits, or call sdpa_fwd with a workspace)",
                                  need, kNoallocScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return sdpa::record_error(SDPA_ERR_DEVICE, "no usable current device (hipGetDevice: %s, device %d)",
                                      hipGetErrorString(e), dev);
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return sdpa::record_error(SDPA_ERR_DEVICE, "hipGetSymbolAddress of the scratch array failed: %s",
                                          hipGetErrorString(e));
            g_scratch_ptr[dev] = p;
        }
        ws = g_scratch_ptr[dev];
    }
    return sdpa_fwd(dtype, q, k, v, attn_mask, mask_dtype, dropout_p, is_causal, scale, enable_gqa, out, lse, ws,
                    ws ? kNoallocScratchBytes : 0, num_splits, stream);
}
