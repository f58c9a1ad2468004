// Prefill with a library-owned workspace, for callers that cannot allocate
// device memory (graph capture, serving loops, harnesses without hipMalloc).
//
// The workspace is the file-scope device array `scratch` below. In host code
// its name is only a host-side stand-in, never a device address: the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that pointer is
// passed on. Nothing here allocates device memory.

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "gdn_internal.h"

namespace {

constexpr size_t kScratchBytes = GDN_PREFILL_STATIC_WORKSPACE_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `dev`'s copy of the array (looked up on first use).
int scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices)
        return gdn::fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked_static: device index " + std::to_string(dev) +
                                                " beyond the library's table");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked_static: hipGetDevice: ") + hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked_static: hipSetDevice: ") + hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess && e2 != hipSuccess) e = e2;
        }
        if (e != hipSuccess || p == nullptr)
            return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked_static: hipGetSymbolAddress: ") +
                                            hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GDN_OK;
}

}  // namespace

extern "C" int gdn_prefill_chunked_static(const gdn_pool* pool, const gdn_prefill_args* a, void* stream) {
    gdn::PrefillPlan plan;
    const int st = gdn::plan_prefill(pool, a, &plan);
    if (st != GDN_OK) return st;
    if (plan.bytes > kScratchBytes)
        return gdn::fail(GDN_E_INVALID, "gdn_prefill_chunked_static: this call needs " + std::to_string(plan.bytes) +
                                            " bytes of workspace, more than the library's static " +
                                            std::to_string(kScratchBytes) +
                                            "; split the call or use gdn_prefill_chunked with a caller workspace");
    if (a->num_seqs == 0) return GDN_OK;
    int dev = -1;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked_static: device of the stream: ") + hipGetErrorString(e));
    void* ws = nullptr;
    const int s2 = scratch_on(dev, &ws);
    if (s2 != GDN_OK) return s2;
    return gdn_prefill_chunked(pool, a, ws, kScratchBytes, stream);
}
