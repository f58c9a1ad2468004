// Recorded decode step: a list of decode launches captured once into a HIP
// graph and replayed per step, closed by a sentinel kernel that reports the
// replay to pinned host memory.
//
// Source: the TokenSpeed article (24-ai.news, English, section "What are the
// key optimizations behind the record?", item "CUDA graph recording") and
// zubnet.ai (Portuguese), second paragraph (graph capture, pinned-memory
// copies, event-based layer barriers, GPU-side sentinels).
//
// The graph holds, in order: every entry's decode kernel (each followed by an
// event record when per-entry events are asked for), then one sentinel kernel.
// Nothing in it clears memory with a memset node: the sentinel kernel clears
// the error word itself.

#include <hip/hip_runtime.h>

#include <atomic>
#include <string>
#include <vector>

#include "gdn_internal.h"

struct gdn_decode_graph {
    int32_t num_entries = 0;
    bool events_on = false;
    std::vector<hipEvent_t> events;          // one per entry when events_on
    uint32_t* replays_dev = nullptr;         // device counter of finished replays
    unsigned long long* word = nullptr;      // pinned host word: (replays << 32) | flags
    unsigned long long* word_dev = nullptr;  // its device address
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

// One thread: count the replay, take and clear the error word, and publish
// both as one 64-bit store to host memory, so the host never sees a count
// without its flags.
__global__ void sentinel_kernel(int32_t* err, uint32_t* replays, unsigned long long* word) {
    if (threadIdx.x != 0) return;
    // Atomic loads keep both reads on the vector memory path.
    const uint32_t n = __hip_atomic_load(replays, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    *replays = n;
    const uint32_t f = static_cast<uint32_t>(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    *err = 0;
    __hip_atomic_store(word, (static_cast<unsigned long long>(n) << 32) | f, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}

int hip_fail(const char* what, hipError_t e) {
    return gdn::fail(GDN_E_HIP, std::string("gdn_decode_graph: ") + what + ": " + hipGetErrorString(e));
}

void release(gdn_decode_graph* g) {
    if (g == nullptr) return;
    if (g->exec != nullptr) (void)hipGraphExecDestroy(g->exec);
    if (g->graph != nullptr) (void)hipGraphDestroy(g->graph);
    for (hipEvent_t e : g->events)
        if (e != nullptr) (void)hipEventDestroy(e);
    if (g->replays_dev != nullptr) (void)hipFree(g->replays_dev);
    if (g->word != nullptr) (void)hipHostFree(g->word);
    delete g;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// Capture every launch on `cs`. Capture is always ended, also after a failed
// launch, so the stream is never left capturing.
int record(gdn_decode_graph* g, const gdn_pool* pool, const gdn_decode_args* entries, float* const* storages,
           hipStream_t cs) {
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail("hipStreamBeginCapture", e);
    int st = GDN_OK;
    for (int32_t i = 0; i < g->num_entries && st == GDN_OK; ++i) {
        float* storage = storages != nullptr ? storages[i] : nullptr;
        st = gdn::launch_decode(pool, &entries[i], cs, storage);
        if (st == GDN_OK && g->events_on) {
            e = hipEventRecord(g->events[static_cast<size_t>(i)], cs);
            if (e != hipSuccess) st = hip_fail("hipEventRecord", e);
        }
    }
    if (st == GDN_OK) {
        hipLaunchKernelGGL(sentinel_kernel, dim3(1), dim3(64), 0, cs, entries[0].err_flag, g->replays_dev,
                           g->word_dev);
        e = hipGetLastError();
        if (e != hipSuccess) st = hip_fail("sentinel launch", e);
    }
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    if (st != GDN_OK) {
        if (graph != nullptr) (void)hipGraphDestroy(graph);
        return st;
    }
    if (e != hipSuccess) return hip_fail("hipStreamEndCapture", e);
    g->graph = graph;
    e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        g->exec = nullptr;
        return hip_fail("hipGraphInstantiate", e);
    }
    return GDN_OK;
}

}  // namespace

extern "C" int gdn_decode_graph_create(const gdn_pool* pool, int32_t num_entries, const gdn_decode_args* entries,
                                       float* const* storages, int32_t flags, gdn_decode_graph** out) {
    using gdn::fail;
    if (pool == nullptr || entries == nullptr || out == nullptr)
        return fail(GDN_E_INVALID, "gdn_decode_graph_create: NULL pool, entries or out");
    if (num_entries < 1 || num_entries > GDN_GRAPH_MAX_ENTRIES)
        return fail(GDN_E_INVALID, "gdn_decode_graph_create: num_entries must be in [1, " +
                                       std::to_string(GDN_GRAPH_MAX_ENTRIES) + "]");
    if (flags != 0 && flags != GDN_GRAPH_LAYER_EVENTS)
        return fail(GDN_E_INVALID, "gdn_decode_graph_create: flags must be 0 or GDN_GRAPH_LAYER_EVENTS");
    for (int32_t i = 0; i < num_entries; ++i) {
        const std::string fn = "gdn_decode_graph_create: entry " + std::to_string(i);
        const int st = gdn::check_decode_args(pool, &entries[i], fn.c_str());
        if (st != GDN_OK) return st;
        if (entries[i].batch < 1) return fail(GDN_E_INVALID, fn + ": batch must be >= 1");
        if (entries[i].err_flag == nullptr || entries[i].err_flag != entries[0].err_flag)
            return fail(GDN_E_INVALID, fn + ": every entry must name the same non-NULL err_flag");
        if (storages != nullptr && storages[i] != nullptr && !aligned16(storages[i]))
            return fail(GDN_E_INVALID, fn + ": storage must be 16-byte aligned");
    }

    auto* g = new gdn_decode_graph();
    g->num_entries = num_entries;
    g->events_on = (flags & GDN_GRAPH_LAYER_EVENTS) != 0;
    hipError_t e;
    if (g->events_on) {
        g->events.assign(static_cast<size_t>(num_entries), nullptr);
        for (auto& ev : g->events) {
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
            if (e != hipSuccess) {
                ev = nullptr;
                release(g);
                return hip_fail("hipEventCreateWithFlags", e);
            }
        }
    }
    e = hipMalloc(reinterpret_cast<void**>(&g->replays_dev), 256);
    if (e != hipSuccess) {
        g->replays_dev = nullptr;
        release(g);
        return hip_fail("hipMalloc", e);
    }
    e = hipMemset(g->replays_dev, 0, 256);  // synchronous, outside any graph
    if (e != hipSuccess) {
        release(g);
        return hip_fail("hipMemset", e);
    }
    e = hipHostMalloc(reinterpret_cast<void**>(&g->word), 64, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) {
        g->word = nullptr;
        release(g);
        return hip_fail("hipHostMalloc", e);
    }
    __atomic_store_n(g->word, 0ull, __ATOMIC_RELEASE);
    e = hipHostGetDevicePointer(reinterpret_cast<void**>(&g->word_dev), g->word, 0);
    if (e != hipSuccess) {
        release(g);
        return hip_fail("hipHostGetDevicePointer", e);
    }

    hipStream_t cs = nullptr;
    e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) {
        release(g);
        return hip_fail("hipStreamCreateWithFlags", e);
    }
    const int st = record(g, pool, entries, storages, cs);
    (void)hipStreamDestroy(cs);
    if (st != GDN_OK) {
        release(g);
        return st;
    }
    *out = g;
    return GDN_OK;
}

extern "C" int gdn_decode_graph_launch(gdn_decode_graph* graph, void* stream) {
    if (graph == nullptr) return gdn::fail(GDN_E_INVALID, "gdn_decode_graph_launch: NULL graph");
    const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("hipGraphLaunch", e);
    return GDN_OK;
}

extern "C" int gdn_decode_graph_poll(const gdn_decode_graph* graph, uint32_t* replays, int32_t* flags) {
    if (graph == nullptr || replays == nullptr || flags == nullptr)
        return gdn::fail(GDN_E_INVALID, "gdn_decode_graph_poll: NULL argument");
    const unsigned long long w = __atomic_load_n(graph->word, __ATOMIC_ACQUIRE);
    *replays = static_cast<uint32_t>(w >> 32);
    *flags = static_cast<int32_t>(static_cast<uint32_t>(w));
    return GDN_OK;
}

static int entry_event(const gdn_decode_graph* graph, int32_t entry, const char* fn, hipEvent_t* ev) {
    if (graph == nullptr) return gdn::fail(GDN_E_INVALID, std::string(fn) + ": NULL graph");
    if (!graph->events_on)
        return gdn::fail(GDN_E_INVALID, std::string(fn) + ": graph was created without GDN_GRAPH_LAYER_EVENTS");
    if (entry < 0 || entry >= graph->num_entries)
        return gdn::fail(GDN_E_INVALID, std::string(fn) + ": entry " + std::to_string(entry) + " out of range");
    *ev = graph->events[static_cast<size_t>(entry)];
    return GDN_OK;
}

extern "C" int gdn_decode_graph_wait_entry(const gdn_decode_graph* graph, int32_t entry, void* stream) {
    hipEvent_t ev = nullptr;
    const int st = entry_event(graph, entry, "gdn_decode_graph_wait_entry", &ev);
    if (st != GDN_OK) return st;
    const hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), ev, 0);
    if (e != hipSuccess) return hip_fail("hipStreamWaitEvent", e);
    return GDN_OK;
}

extern "C" int gdn_decode_graph_sync_entry(const gdn_decode_graph* graph, int32_t entry) {
    hipEvent_t ev = nullptr;
    const int st = entry_event(graph, entry, "gdn_decode_graph_sync_entry", &ev);
    if (st != GDN_OK) return st;
    const hipError_t e = hipEventSynchronize(ev);
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
    return GDN_OK;
}

extern "C" int gdn_decode_graph_destroy(gdn_decode_graph* graph) {
    if (graph == nullptr) return GDN_OK;
    // A replay still in flight would write the host word and read the
    // events; let the device drain before freeing them.
    const hipError_t e = hipDeviceSynchronize();
    release(graph);
    if (e != hipSuccess) return hip_fail("hipDeviceSynchronize", e);
    return GDN_OK;
}
