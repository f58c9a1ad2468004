// Slot pack / unpack for state transfer (gfx950).
//
// The prefill-decode split of the TokenSpeed engine hands a request's state
// from one phase to the other (24-ai.news, English, section "What are the key
// optimizations behind the record?", item "Prefill-Decode disaggregation").
// On one GPU that hand-over is a gather of slot tiles into a contiguous buffer
// (pack) and the scatter back into slots (unpack): a streaming copy, bound by
// HBM bandwidth. One workgroup per (entry, value head) tile, 128-bit
// non-temporal loads and stores (each tile is touched once).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gdn_internal.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

struct TransferParams {
    float* pool;
    float* buf;               // [n][HV][tile]
    const int32_t* slots;
    int32_t* err;
    int32_t hv;
    int32_t num_slots;
    int32_t tile_f4;          // dk * dv / 4
};

template <bool PACK>
__global__ void __launch_bounds__(kThreads) transfer_kernel(TransferParams p) {
    const int e = blockIdx.x / p.hv;
    const int h = blockIdx.x - e * p.hv;
    const int s = p.slots[e];
    if (s >= p.num_slots) {
        if (threadIdx.x == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
        return;
    }
    if (!PACK && s < 0) return;          // unpack skips negative entries
    f4* b = reinterpret_cast<f4*>(p.buf) + static_cast<size_t>(blockIdx.x) * p.tile_f4;
    f4* t = s >= 0 ? reinterpret_cast<f4*>(p.pool) + (static_cast<size_t>(s) * p.hv + h) * p.tile_f4 : nullptr;
    for (int i = threadIdx.x; i < p.tile_f4; i += kThreads) {
        if (PACK)
            __builtin_nontemporal_store(t != nullptr ? __builtin_nontemporal_load(t + i) : f4{0.f, 0.f, 0.f, 0.f}, b + i);
        else
            __builtin_nontemporal_store(__builtin_nontemporal_load(b + i), t + i);
    }
}

}  // namespace

namespace gdn {

int launch_transfer(const gdn_pool* pool, bool pack, int32_t n, const int32_t* slots, float* buffer,
                    int32_t* err_flag, void* stream) {
    TransferParams p;
    p.pool = pool->storage;
    p.buf = buffer;
    p.slots = slots;
    p.err = err_flag;
    p.hv = pool->num_v_heads;
    p.num_slots = pool->num_slots;
    p.tile_f4 = pool->dk * pool->dv / 4;
    const dim3 grid(static_cast<unsigned>(n) * static_cast<unsigned>(pool->num_v_heads));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pack) hipLaunchKernelGGL(transfer_kernel<true>, grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(transfer_kernel<false>, grid, dim3(kThreads), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(GDN_E_HIP, std::string(pack ? "gdn_state_pool_pack" : "gdn_state_pool_unpack") +
                                   ": launch failed: " + hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace gdn
