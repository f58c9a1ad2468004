// Host bookkeeping of the state-slot pool, and the library's error channel.
//
// A slot is one fixed-size recurrent state (HV tiles of dk x dv float32) in
// caller-owned device memory. The pool only counts references: it never reads
// or writes state bytes. Reuse of a cached checkpoint is copy-on-write and
// advancing a request is an index update, never a copy -- the slot reuse and
// index indirection described in the TokenSpeed article (24-ai.news, English),
// section "What are the key optimizations behind the record?", items "Hybrid
// prefix caching for GDN/Mamba" and "Mamba State Update optimization".

#include <cstdint>
#include <new>
#include <string>
#include <unordered_set>

#include "gdn_internal.h"

namespace gdn {

static thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

}  // namespace gdn

using gdn::fail;

static bool valid_head_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

extern "C" const char* gdn_last_error(void) { return gdn::g_last_error.c_str(); }

extern "C" int gdn_state_pool_create(int32_t num_slots, int32_t num_v_heads, int32_t dk, int32_t dv,
                                     float* storage, gdn_pool** out) {
    if (out == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_create: out is NULL");
    if (num_slots <= 0) return fail(GDN_E_INVALID, "gdn_state_pool_create: num_slots must be > 0");
    if (num_v_heads <= 0) return fail(GDN_E_INVALID, "gdn_state_pool_create: num_v_heads must be > 0");
    if (!valid_head_dim(dk) || !valid_head_dim(dv))
        return fail(GDN_E_INVALID, "gdn_state_pool_create: dk and dv must be 16, 32, 64 or 128");
    if (storage == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_create: storage is NULL");
    if (reinterpret_cast<uintptr_t>(storage) % 16 != 0)
        return fail(GDN_E_INVALID, "gdn_state_pool_create: storage must be 16-byte aligned");
    gdn_pool* p = new (std::nothrow) gdn_pool();
    if (p == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_create: out of host memory");
    p->num_slots = num_slots;
    p->num_v_heads = num_v_heads;
    p->dk = dk;
    p->dv = dv;
    p->storage = storage;
    p->ref.assign(static_cast<size_t>(num_slots), 0);
    for (int32_t i = 0; i < num_slots; ++i) p->free_slots.insert(p->free_slots.end(), i);
    *out = p;
    return GDN_OK;
}

extern "C" int gdn_state_pool_destroy(gdn_pool* pool) {
    delete pool;
    return GDN_OK;
}

extern "C" int gdn_state_pool_alloc(gdn_pool* pool, int32_t n, int32_t* out) {
    if (pool == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_alloc: pool is NULL");
    if (n < 0) return fail(GDN_E_INVALID, "gdn_state_pool_alloc: n must be >= 0");
    if (n > 0 && out == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_alloc: out is NULL");
    if (static_cast<size_t>(n) > pool->free_slots.size())
        return fail(GDN_E_NO_SLOTS, "gdn_state_pool_alloc: requested " + std::to_string(n) + " slots, " +
                                        std::to_string(pool->free_slots.size()) + " free");
    for (int32_t i = 0; i < n; ++i) {
        auto it = pool->free_slots.begin();
        const int32_t s = *it;
        pool->free_slots.erase(it);
        pool->ref[static_cast<size_t>(s)] = 1;
        out[i] = s;
    }
    return GDN_OK;
}

static int check_slot(const gdn_pool* pool, int32_t slot, const char* fn) {
    if (pool == nullptr) return fail(GDN_E_INVALID, std::string(fn) + ": pool is NULL");
    if (slot < 0 || slot >= pool->num_slots)
        return fail(GDN_E_INVALID, std::string(fn) + ": slot " + std::to_string(slot) + " out of range");
    if (pool->ref[static_cast<size_t>(slot)] == 0)
        return fail(GDN_E_SLOT_STATE, std::string(fn) + ": slot " + std::to_string(slot) + " is free");
    return GDN_OK;
}

extern "C" int gdn_state_pool_retain(gdn_pool* pool, int32_t slot) {
    const int st = check_slot(pool, slot, "gdn_state_pool_retain");
    if (st != GDN_OK) return st;
    pool->ref[static_cast<size_t>(slot)] += 1;
    return GDN_OK;
}

extern "C" int gdn_state_pool_release(gdn_pool* pool, int32_t slot) {
    const int st = check_slot(pool, slot, "gdn_state_pool_release");
    if (st != GDN_OK) return st;
    if (--pool->ref[static_cast<size_t>(slot)] == 0) pool->free_slots.insert(slot);
    return GDN_OK;
}

extern "C" int gdn_state_pool_cow(gdn_pool* pool, int32_t src, int32_t* dst) {
    if (pool == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_cow: pool is NULL");
    if (dst == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_cow: dst is NULL");
    if (src >= pool->num_slots)
        return fail(GDN_E_INVALID, "gdn_state_pool_cow: slot " + std::to_string(src) + " out of range");
    if (src >= 0) {
        const int32_t r = pool->ref[static_cast<size_t>(src)];
        if (r == 0) return fail(GDN_E_SLOT_STATE, "gdn_state_pool_cow: slot " + std::to_string(src) + " is free");
        if (r == 1) {
            *dst = src;
            return GDN_OK;
        }
    }
    int32_t fresh = -1;
    const int st = gdn_state_pool_alloc(pool, 1, &fresh);
    if (st != GDN_OK) return st;
    *dst = fresh;
    return GDN_OK;
}

extern "C" int gdn_state_pool_validate(const gdn_pool* pool, int32_t n, const int32_t* src_host,
                                       const int32_t* dst_host) {
    if (pool == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_validate: pool is NULL");
    if (n < 0) return fail(GDN_E_INVALID, "gdn_state_pool_validate: n must be >= 0");
    if (n > 0 && (src_host == nullptr || dst_host == nullptr))
        return fail(GDN_E_INVALID, "gdn_state_pool_validate: NULL table");
    for (int32_t i = 0; i < n; ++i) {
        const int32_t pair[2] = {src_host[i], dst_host[i]};
        for (int32_t x : pair) {
            if (x >= pool->num_slots)
                return fail(GDN_E_INVALID, "gdn_state_pool_validate: entry " + std::to_string(i) + " slot " +
                                               std::to_string(x) + " out of range");
            if (x >= 0 && pool->ref[static_cast<size_t>(x)] == 0)
                return fail(GDN_E_SLOT_STATE, "gdn_state_pool_validate: entry " + std::to_string(i) + " slot " +
                                                  std::to_string(x) + " is free");
        }
    }
    std::unordered_set<int32_t> dsts;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t d = dst_host[i];
        if (d >= 0 && !dsts.insert(d).second)
            return fail(GDN_E_ALIAS, "gdn_state_pool_validate: destination " + std::to_string(d) + " repeated");
    }
    // A destination may equal its own entry's source (in place) but no other
    // entry's source: that entry would read bytes this one overwrites.
    std::unordered_multiset<int32_t> srcs;
    for (int32_t i = 0; i < n; ++i)
        if (src_host[i] >= 0) srcs.insert(src_host[i]);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t d = dst_host[i];
        if (d < 0) continue;
        const size_t uses = srcs.count(d);
        if (uses > (src_host[i] == d ? 1u : 0u))
            return fail(GDN_E_ALIAS, "gdn_state_pool_validate: destination " + std::to_string(d) +
                                         " is another entry's source");
    }
    return GDN_OK;
}

extern "C" int gdn_state_pool_refcount(const gdn_pool* pool, int32_t slot, int32_t* out) {
    if (pool == nullptr || out == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_refcount: NULL argument");
    if (slot < 0 || slot >= pool->num_slots)
        return fail(GDN_E_INVALID, "gdn_state_pool_refcount: slot " + std::to_string(slot) + " out of range");
    *out = pool->ref[static_cast<size_t>(slot)];
    return GDN_OK;
}

extern "C" int gdn_state_pool_num_free(const gdn_pool* pool, int32_t* out) {
    if (pool == nullptr || out == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_num_free: NULL argument");
    *out = static_cast<int32_t>(pool->free_slots.size());
    return GDN_OK;
}

extern "C" int gdn_state_pool_capacity(const gdn_pool* pool, int32_t* out) {
    if (pool == nullptr || out == nullptr) return fail(GDN_E_INVALID, "gdn_state_pool_capacity: NULL argument");
    *out = pool->num_slots;
    return GDN_OK;
}
