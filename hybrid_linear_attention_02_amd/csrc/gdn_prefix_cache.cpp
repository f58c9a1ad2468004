// Prefix cache: a radix tree over token ids whose nodes own slot checkpoints.
//
// The logical half of the hybrid prefix caching on the TokenSpeed pages
// (24-ai.news, English, section "What are the key optimizations behind the
// record?", item "Hybrid prefix caching for GDN/Mamba"): the tree decides
// which stored linear-attention state a new request can resume from; the
// states themselves live in pool slots (device memory) and are only ever
// referenced here through the pool's refcounts.
//
// Edges carry runs of tokens (a compressed trie). A node at depth d may own
// the checkpoint of the d-token prefix that ends there. Recency is a logical
// clock stamped on insert and on every hit; eviction takes the oldest
// checkpoint whose slot nobody else holds.

#include <algorithm>
#include <cstdint>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "gdn_internal.h"

using gdn::fail;

namespace {

struct Node {
    std::vector<int32_t> edge;                       // tokens from the parent to this node
    std::map<int32_t, std::unique_ptr<Node>> kids;   // keyed by the first token of the child's edge
    Node* parent = nullptr;
    int64_t depth = 0;                               // prefix length at this node
    int32_t slot = -1;                               // checkpoint slot, -1 = none
    uint64_t used = 0;                               // recency stamp of the checkpoint
};

int32_t refcount_of(const gdn_pool* pool, int32_t slot) {
    int32_t r = 0;
    gdn_state_pool_refcount(pool, slot, &r);
    return r;
}

}  // namespace

struct gdn_prefix_cache {
    gdn_pool* pool = nullptr;
    Node root;
    uint64_t clock = 0;
    int32_t count = 0;
};

namespace {

// Remove `node` if it owns nothing and leads nowhere (and so on upwards),
// then splice out a node left with no checkpoint and a single child: the
// child moves up to the grandparent with the two edges joined (keeps the tree
// compressed). Only nodes without a checkpoint are destroyed; the objects of
// nodes that own one never move, so pointers to them stay valid.
void prune(gdn_prefix_cache* c, Node* node) {
    while (node != &c->root && node->slot < 0 && node->kids.empty()) {
        Node* parent = node->parent;
        parent->kids.erase(node->edge.front());
        node = parent;
    }
    if (node != &c->root && node->slot < 0 && node->kids.size() == 1) {
        Node* parent = node->parent;
        std::unique_ptr<Node> child = std::move(node->kids.begin()->second);
        child->edge.insert(child->edge.begin(), node->edge.begin(), node->edge.end());
        child->parent = parent;
        const int32_t key = child->edge.front();
        parent->kids[key] = std::move(child);            // destroys `node`
    }
}

// Every node below `root` (iteratively: a long chain of prefixes must not
// exhaust the stack).
std::vector<Node*> all_nodes(Node* root) {
    std::vector<Node*> out, todo{root};
    while (!todo.empty()) {
        Node* n = todo.back();
        todo.pop_back();
        out.push_back(n);
        for (auto& kv : n->kids) todo.push_back(kv.second.get());
    }
    return out;
}

}  // namespace

extern "C" int gdn_prefix_cache_create(gdn_pool* pool, gdn_prefix_cache** out) {
    if (pool == nullptr || out == nullptr) return fail(GDN_E_INVALID, "gdn_prefix_cache_create: NULL argument");
    auto* c = new gdn_prefix_cache();
    c->pool = pool;
    *out = c;
    return GDN_OK;
}

extern "C" int gdn_prefix_cache_destroy(gdn_prefix_cache* cache) {
    if (cache == nullptr) return GDN_OK;
    // release the references, then free the nodes leaf-first without recursion
    std::vector<std::unique_ptr<Node>> owned;
    std::vector<Node*> todo{&cache->root};
    while (!todo.empty()) {
        Node* n = todo.back();
        todo.pop_back();
        if (n->slot >= 0) gdn_state_pool_release(cache->pool, n->slot);
        for (auto& kv : n->kids) {
            todo.push_back(kv.second.get());
            owned.push_back(std::move(kv.second));
        }
        n->kids.clear();
    }
    owned.clear();
    delete cache;
    return GDN_OK;
}

extern "C" int gdn_prefix_cache_insert(gdn_prefix_cache* c, const int32_t* tokens, int32_t n, int32_t slot,
                                       int32_t* inserted) {
    if (c == nullptr || tokens == nullptr || inserted == nullptr)
        return fail(GDN_E_INVALID, "gdn_prefix_cache_insert: NULL argument");
    if (n <= 0) return fail(GDN_E_INVALID, "gdn_prefix_cache_insert: n must be > 0");
    if (slot < 0 || slot >= c->pool->num_slots)
        return fail(GDN_E_INVALID, "gdn_prefix_cache_insert: slot " + std::to_string(slot) + " out of range");
    if (refcount_of(c->pool, slot) == 0)
        return fail(GDN_E_SLOT_STATE, "gdn_prefix_cache_insert: slot " + std::to_string(slot) + " is free");
    Node* node = &c->root;
    int32_t i = 0;
    while (i < n) {
        auto it = node->kids.find(tokens[i]);
        if (it == node->kids.end()) {                 // a new leaf carries the rest
            auto leaf = std::make_unique<Node>();
            leaf->edge.assign(tokens + i, tokens + n);
            leaf->parent = node;
            leaf->depth = n;
            Node* raw = leaf.get();
            node->kids.emplace(tokens[i], std::move(leaf));
            node = raw;
            i = n;
            break;
        }
        Node* child = it->second.get();
        const int32_t room = static_cast<int32_t>(child->edge.size());
        int32_t m = 0;
        while (m < room && i + m < n && child->edge[m] == tokens[i + m]) ++m;
        if (m == room) {                              // the whole edge matches
            node = child;
            i += m;
            continue;
        }
        // split the edge after m tokens: parent -> mid -> child
        auto mid = std::make_unique<Node>();
        mid->edge.assign(child->edge.begin(), child->edge.begin() + m);
        mid->parent = node;
        mid->depth = node->depth + m;
        std::unique_ptr<Node> moved = std::move(it->second);
        moved->edge.erase(moved->edge.begin(), moved->edge.begin() + m);
        moved->parent = mid.get();
        const int32_t key = moved->edge.front();
        mid->kids.emplace(key, std::move(moved));
        Node* raw = mid.get();
        it->second = std::move(mid);
        node = raw;
        i += m;
    }
    if (node->slot >= 0) {
        *inserted = 0;
        return GDN_OK;
    }
    const int st = gdn_state_pool_retain(c->pool, slot);
    if (st != GDN_OK) {
        prune(c, node);
        return st;
    }
    node->slot = slot;
    node->used = ++c->clock;
    ++c->count;
    *inserted = 1;
    return GDN_OK;
}

extern "C" int gdn_prefix_cache_match(gdn_prefix_cache* c, const int32_t* tokens, int32_t n, int32_t* len,
                                      int32_t* slot) {
    if (c == nullptr || len == nullptr || slot == nullptr || (tokens == nullptr && n > 0))
        return fail(GDN_E_INVALID, "gdn_prefix_cache_match: NULL argument");
    if (n < 0) return fail(GDN_E_INVALID, "gdn_prefix_cache_match: n must be >= 0");
    Node* node = &c->root;
    Node* best = nullptr;
    int32_t i = 0;
    while (i < n) {
        auto it = node->kids.find(tokens[i]);
        if (it == node->kids.end()) break;
        Node* child = it->second.get();
        const int32_t room = static_cast<int32_t>(child->edge.size());
        if (i + room > n || !std::equal(child->edge.begin(), child->edge.end(), tokens + i)) break;
        node = child;
        i += room;
        if (node->slot >= 0) best = node;
    }
    if (best == nullptr) {
        *len = 0;
        *slot = -1;
        return GDN_OK;
    }
    const int st = gdn_state_pool_retain(c->pool, best->slot);
    if (st != GDN_OK) return st;
    best->used = ++c->clock;
    *len = static_cast<int32_t>(best->depth);
    *slot = best->slot;
    return GDN_OK;
}

extern "C" int gdn_prefix_cache_evict(gdn_prefix_cache* c, int32_t want_free, int32_t* dropped) {
    if (c == nullptr || dropped == nullptr) return fail(GDN_E_INVALID, "gdn_prefix_cache_evict: NULL argument");
    std::vector<Node*> held;
    for (Node* node : all_nodes(&c->root))
        if (node->slot >= 0) held.push_back(node);
    std::sort(held.begin(), held.end(), [](const Node* a, const Node* b) { return a->used < b->used; });
    int32_t n = 0;
    for (Node* node : held) {
        int32_t free_now = 0;
        gdn_state_pool_num_free(c->pool, &free_now);
        if (free_now >= want_free) break;
        if (refcount_of(c->pool, node->slot) != 1) continue;   // someone else still reads it
        gdn_state_pool_release(c->pool, node->slot);
        node->slot = -1;
        --c->count;
        ++n;
        prune(c, node);
    }
    *dropped = n;
    return GDN_OK;
}

extern "C" int gdn_prefix_cache_size(const gdn_prefix_cache* c, int32_t* out) {
    if (c == nullptr || out == nullptr) return fail(GDN_E_INVALID, "gdn_prefix_cache_size: NULL argument");
    *out = c->count;
    return GDN_OK;
}
