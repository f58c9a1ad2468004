// Argument checking and dispatch of the launching entry points.
//
// Everything here runs on the host before any work is enqueued: a call that
// fails a check returns a GDN_E_* code with a message and enqueues nothing.
// Slot tables live in device memory and are not read here (that would need a
// device-to-host round trip); gdn_state_pool_validate checks a host copy, and
// the kernels skip and flag out-of-range indices.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "gdn_internal.h"

using gdn::fail;

static bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

static int check_heads(const gdn_pool* pool, int32_t hk, int32_t hv, int32_t dk, int32_t dv, const char* fn) {
    if (hk <= 0 || hv <= 0 || hv % hk != 0)
        return fail(GDN_E_INVALID, std::string(fn) + ": num_v_heads must be a positive multiple of num_k_heads");
    if (hv != pool->num_v_heads || dk != pool->dk || dv != pool->dv)
        return fail(GDN_E_INVALID, std::string(fn) + ": head shape does not match the pool (HV " +
                                       std::to_string(pool->num_v_heads) + ", dk " + std::to_string(pool->dk) +
                                       ", dv " + std::to_string(pool->dv) + ")");
    return GDN_OK;
}

static int transfer(const gdn_pool* pool, bool pack, int32_t n, const int32_t* slots, const float* buffer,
                    int32_t* err_flag, void* stream) {
    const std::string fn = pack ? "gdn_state_pool_pack" : "gdn_state_pool_unpack";
    if (pool == nullptr) return fail(GDN_E_INVALID, fn + ": NULL pool");
    if (n < 0) return fail(GDN_E_INVALID, fn + ": n must be >= 0");
    if (static_cast<int64_t>(n) * pool->num_v_heads > INT32_MAX) return fail(GDN_E_INVALID, fn + ": n too large");
    if (n == 0) return GDN_OK;
    if (slots == nullptr || buffer == nullptr) return fail(GDN_E_INVALID, fn + ": NULL slot table or buffer");
    if (!aligned(buffer, 16)) return fail(GDN_E_INVALID, fn + ": buffer must be 16-byte aligned");
    if (!aligned(slots, 4) || !aligned(err_flag, 4)) return fail(GDN_E_INVALID, fn + ": slots, err_flag must be 4-byte aligned");
    return gdn::launch_transfer(pool, pack, n, slots, const_cast<float*>(buffer), err_flag, stream);
}

extern "C" int gdn_state_pool_pack(const gdn_pool* pool, int32_t n, const int32_t* slots, float* buffer,
                                   int32_t* err_flag, void* stream) {
    return transfer(pool, true, n, slots, buffer, err_flag, stream);
}

extern "C" int gdn_state_pool_unpack(const gdn_pool* pool, int32_t n, const int32_t* slots, const float* buffer,
                                     int32_t* err_flag, void* stream) {
    return transfer(pool, false, n, slots, buffer, err_flag, stream);
}

namespace gdn {

// Checks of one decode step's arguments, shared by gdn_decode_step and the
// recorded decode graph. GDN_OK for batch == 0 without looking at pointers.
int check_decode_args(const gdn_pool* pool, const gdn_decode_args* a, const char* fn) {
    if (pool == nullptr || a == nullptr) return fail(GDN_E_INVALID, std::string(fn) + ": NULL pool or args");
    if (a->batch < 0) return fail(GDN_E_INVALID, std::string(fn) + ": batch must be >= 0");
    const int st = check_heads(pool, a->num_k_heads, a->num_v_heads, a->dk, a->dv, fn);
    if (st != GDN_OK) return st;
    if (a->dtype != GDN_DTYPE_F32 && a->dtype != GDN_DTYPE_BF16)
        return fail(GDN_E_UNSUPPORTED, std::string(fn) + ": dtype must be GDN_DTYPE_F32 or GDN_DTYPE_BF16");
    if (!std::isfinite(a->scale) || !(a->l2_eps >= 0.0f) || !std::isfinite(a->l2_eps))
        return fail(GDN_E_INVALID, std::string(fn) + ": scale must be finite and l2_eps finite and >= 0");
    if (static_cast<int64_t>(a->batch) * a->num_v_heads > INT32_MAX)
        return fail(GDN_E_INVALID, std::string(fn) + ": batch * num_v_heads too large");
    if (a->batch == 0) return GDN_OK;
    const void* ptrs[] = {a->q, a->k, a->v, a->g, a->beta, a->o, a->src_slots, a->dst_slots};
    for (const void* p : ptrs)
        if (p == nullptr) return fail(GDN_E_INVALID, std::string(fn) + ": NULL device pointer");
    const void* vec[] = {a->q, a->k, a->v, a->o};
    for (const void* p : vec)
        if (!aligned(p, 16)) return fail(GDN_E_INVALID, std::string(fn) + ": q, k, v, o must be 16-byte aligned");
    const void* word[] = {a->g, a->beta, a->src_slots, a->dst_slots, a->err_flag};
    for (const void* p : word)
        if (!aligned(p, 4)) return fail(GDN_E_INVALID, std::string(fn) + ": g, beta, slot tables, err_flag must be 4-byte aligned");
    return GDN_OK;
}

}  // namespace gdn

extern "C" int gdn_decode_step(const gdn_pool* pool, const gdn_decode_args* a, void* stream) {
    const int st = gdn::check_decode_args(pool, a, "gdn_decode_step");
    if (st != GDN_OK || a->batch == 0) return st;
    return gdn::launch_decode(pool, a, stream);
}

extern "C" int gdn_decode_verify(const gdn_pool* pool, const gdn_verify_args* a, void* stream) {
    const char* fn = "gdn_decode_verify";
    if (pool == nullptr || a == nullptr) return fail(GDN_E_INVALID, "gdn_decode_verify: NULL pool or args");
    if (a->batch < 0) return fail(GDN_E_INVALID, "gdn_decode_verify: batch must be >= 0");
    if (a->num_draft < 1 || a->num_draft > gdn::kMaxDraft)
        return fail(GDN_E_INVALID, "gdn_decode_verify: num_draft must be in [1, " + std::to_string(gdn::kMaxDraft) + "]");
    int st = check_heads(pool, a->num_k_heads, a->num_v_heads, a->dk, a->dv, fn);
    if (st != GDN_OK) return st;
    if (a->dtype != GDN_DTYPE_F32 && a->dtype != GDN_DTYPE_BF16)
        return fail(GDN_E_UNSUPPORTED, "gdn_decode_verify: dtype must be GDN_DTYPE_F32 or GDN_DTYPE_BF16");
    if (!std::isfinite(a->scale) || !(a->l2_eps >= 0.0f) || !std::isfinite(a->l2_eps))
        return fail(GDN_E_INVALID, "gdn_decode_verify: scale must be finite and l2_eps finite and >= 0");
    if (static_cast<int64_t>(a->batch) * a->num_v_heads > INT32_MAX ||
        static_cast<int64_t>(a->batch) * a->num_draft * a->num_v_heads * std::max(a->dk, a->dv) > INT32_MAX)
        return fail(GDN_E_INVALID, "gdn_decode_verify: batch too large");
    if (a->batch == 0) return GDN_OK;
    const void* ptrs[] = {a->q, a->k, a->v, a->g, a->beta, a->o, a->src_slots, a->dst_slots};
    for (const void* p : ptrs)
        if (p == nullptr) return fail(GDN_E_INVALID, "gdn_decode_verify: NULL device pointer");
    const void* vec[] = {a->q, a->k, a->v, a->o};
    for (const void* p : vec)
        if (!aligned(p, 16)) return fail(GDN_E_INVALID, "gdn_decode_verify: q, k, v, o must be 16-byte aligned");
    const void* word[] = {a->g, a->beta, a->src_slots, a->dst_slots, a->draft_lens, a->err_flag};
    for (const void* p : word)
        if (!aligned(p, 4))
            return fail(GDN_E_INVALID, "gdn_decode_verify: g, beta, slot tables, draft_lens, err_flag must be 4-byte aligned");
    return gdn::launch_verify(pool, a, stream);
}

extern "C" int gdn_prefill_workspace_bytes(const gdn_pool* pool, const gdn_prefill_args* a, size_t* bytes) {
    if (bytes == nullptr) return fail(GDN_E_INVALID, "gdn_prefill_workspace_bytes: bytes is NULL");
    gdn::PrefillPlan plan;
    const int st = gdn::plan_prefill(pool, a, &plan);
    if (st != GDN_OK) return st;
    *bytes = plan.bytes;
    return GDN_OK;
}

namespace gdn {

static bool prefill_dims_supported(int32_t dk, int32_t dv) {
    return (dk == 16 || dk == 32 || dk == 64 || dk == 128) && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
}

// Segment length of the sequence split, from a cost model of the three
// recurrence passes: a pass takes whole rounds of kNumCUs workgroups (one
// resident per CU), each round as many steps as its longest chain. Costs per
// step are measured cycle counts of the MI355X kernels: state pass 2800 (per
// chunk), output pass 3800 (per chunk, one extra step), 6000 per transition
// the output pass's later segments apply before their first chunk (segment k
// applies k - 1 of them; the first segment runs from the true initial state
// in the state pass, value columns only, so the second needs none). Returns 0
// (no split) when one pass is estimated fastest.
int32_t choose_seg_len(const int32_t* cu, int32_t n, int32_t hv, int32_t dk, int32_t dv) {
    constexpr double kState = 2800, kOut = 3800, kHop = 6000;
    const int nvo = 16 * prefill_output_waves(dv), nvs = 16 * prefill_state_waves(dk, dv);
    const int64_t w_out = static_cast<int64_t>(hv) * (dv / nvo);               // workgroups per segment, output pass
    const int64_t w_val = static_cast<int64_t>(hv) * (dv / nvs);               // state pass, first segment
    const int64_t w_state = static_cast<int64_t>(hv) * ((dv + dk) / nvs);      // state pass, later segments
    auto pass = [](int64_t wg_steps, int64_t longest) {
        // whole rounds of kNumCUs workgroups, each at least `longest` steps
        const double rounds = std::ceil(static_cast<double>(wg_steps) / (static_cast<double>(kNumCUs) * longest));
        return std::max(1.0, rounds) * longest;
    };
    auto cost = [&](int64_t L) {
        int64_t out_steps = 0, state_steps = 0, longest = 0, hops = 0;
        for (int32_t i = 0; i < n; ++i) {
            const int64_t c = (static_cast<int64_t>(cu[i + 1]) - cu[i] + 63) / 64;
            if (c == 0) continue;
            const int64_t nseg = (L == 0 || c <= L) ? 1 : (c + L - 1) / L;
            const int64_t seg = (nseg == 1) ? c : L;
            out_steps += (c + nseg) * w_out;
            if (nseg > 1) state_steps += L * w_val + (nseg - 2) * L * w_state;
            longest = std::max(longest, seg + 1);
            hops = std::max(hops, nseg - 1);
        }
        if (longest == 0) return 0.0;
        double t = kOut * pass(out_steps, longest);
        if (hops > 0) t += kState * pass(state_steps, L) + kHop * static_cast<double>(hops - 1);
        return t;
    };
    // candidates: the longest sequence cut into k equal segments, k = 2 .. 32
    int64_t cmax = 0;
    for (int32_t i = 0; i < n; ++i) cmax = std::max<int64_t>(cmax, (static_cast<int64_t>(cu[i + 1]) - cu[i] + 63) / 64);
    int32_t best = 0;
    double best_cost = cost(0);
    for (int64_t k = 2; k <= 32; ++k) {
        const int64_t L = (cmax + k - 1) / k;
        if (L < 8) break;
        const double c = cost(L);
        if (c < 0.97 * best_cost) {
            best = static_cast<int32_t>(L);
            best_cost = c;
        }
    }
    return best;
}

int plan_prefill(const gdn_pool* pool, const gdn_prefill_args* a, PrefillPlan* plan) {
    const char* fn = "gdn_prefill_chunked";
    if (pool == nullptr || a == nullptr) return fail(GDN_E_INVALID, "gdn_prefill_chunked: NULL pool or args");
    if (a->num_seqs < 0 || a->total_tokens < 0)
        return fail(GDN_E_INVALID, "gdn_prefill_chunked: num_seqs and total_tokens must be >= 0");
    int st = check_heads(pool, a->num_k_heads, a->num_v_heads, a->dk, a->dv, fn);
    if (st != GDN_OK) return st;
    if (a->chunk_size != 64) return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: chunk_size must be 64");
    const bool f32 = a->dtype == GDN_DTYPE_F32;   // chunked form on the fp32 MFMA, any pool head shape
    if (a->dtype != GDN_DTYPE_BF16 && !f32)
        return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: dtype must be GDN_DTYPE_BF16 or GDN_DTYPE_F32");
    if (!f32 && !prefill_dims_supported(a->dk, a->dv))
        return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: dk and dv must be 16, 32, 64 or 128");
    if (!std::isfinite(a->scale) || !(a->l2_eps >= 0.0f) || !std::isfinite(a->l2_eps))
        return fail(GDN_E_INVALID, "gdn_prefill_chunked: scale must be finite and l2_eps finite and >= 0");
    const int32_t n = a->num_seqs;
    if (n > 65535) return fail(GDN_E_INVALID, "gdn_prefill_chunked: at most 65535 sequences per call");
    int64_t chunks = 0, max_chunks = 0;
    if (n > 0) {
        if (a->cu_seqlens_host == nullptr || a->cu_seqlens == nullptr)
            return fail(GDN_E_INVALID, "gdn_prefill_chunked: cu_seqlens (device and host mirror) required");
        if (a->cu_seqlens_host[0] != 0) return fail(GDN_E_INVALID, "gdn_prefill_chunked: cu_seqlens[0] must be 0");
        for (int32_t i = 0; i < n; ++i) {
            const int64_t len = static_cast<int64_t>(a->cu_seqlens_host[i + 1]) - a->cu_seqlens_host[i];
            if (len < 0) return fail(GDN_E_INVALID, "gdn_prefill_chunked: cu_seqlens must be non-decreasing");
            chunks += (len + 63) / 64;
            max_chunks = std::max<int64_t>(max_chunks, (len + 63) / 64);
        }
        if (a->cu_seqlens_host[n] != a->total_tokens)
            return fail(GDN_E_INVALID, "gdn_prefill_chunked: cu_seqlens[N] != total_tokens");
    } else if (a->total_tokens != 0) {
        return fail(GDN_E_INVALID, "gdn_prefill_chunked: total_tokens must be 0 when num_seqs is 0");
    }
    if (chunks * a->num_v_heads > INT32_MAX / 2)
        return fail(GDN_E_INVALID, "gdn_prefill_chunked: too many chunks");
    plan->num_chunks = static_cast<int32_t>(chunks);
    const bool can_split = !f32;
    const int32_t kdk = f32 ? a->dk : prefill_kernel_dk(a->dk);   // the kernels' dk (workspace tiles)
    plan->seg_len = can_split ? choose_seg_len(a->cu_seqlens_host, n, a->num_v_heads, kdk, a->dv) : 0;
    int64_t segs = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t c = (static_cast<int64_t>(a->cu_seqlens_host[i + 1]) - a->cu_seqlens_host[i] + 63) / 64;
        segs += (plan->seg_len == 0 || c <= plan->seg_len) ? 1 : (c + plan->seg_len - 1) / plan->seg_len;
    }
    if (segs > 65535) return fail(GDN_E_INVALID, "gdn_prefill_chunked: too many sequence segments");
    plan->num_segs = static_cast<int32_t>(segs);
    const bool split = plan->seg_len > 0;
    const size_t hv = static_cast<size_t>(a->num_v_heads), dk = static_cast<size_t>(kdk), dv = static_cast<size_t>(a->dv);
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    size_t off = 0;
    plan->off_chunk_offsets = off;
    off = up(off + sizeof(int32_t) * static_cast<size_t>(n + 1));
    plan->off_seg_offsets = off;
    off = up(off + sizeof(int32_t) * static_cast<size_t>(n + 1));
    plan->off_tp = off;
    // T and P per (chunk, value head): bf16 64 x 64 each, or fp32 as the ten
    // lower 16 x 16 blocks each
    off = up(off + (f32 ? 4ull * chunks * hv * 2 * (10 * 64 * 4) : 2ull * chunks * hv * 2 * 64 * 64));
    plan->off_sc = off;
    off = up(off + 4ull * chunks * hv * (5 * 64));
    plan->off_se = off;
    off = up(off + (split ? 4ull * segs * hv * dk * dv : 0));
    plan->off_sm = off;
    off = up(off + (split ? 2ull * segs * hv * 2 * dk * dk : 0));
    plan->off_sh = off;
    off = up(off + (split ? 4ull * segs * hv * dk * dv : 0));
    plan->bytes = off;
    return GDN_OK;
}

}  // namespace gdn

extern "C" int gdn_prefill_chunked(const gdn_pool* pool, const gdn_prefill_args* a, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    gdn::PrefillPlan plan;
    int st = gdn::plan_prefill(pool, a, &plan);
    if (st != GDN_OK) return st;
    if (a->num_seqs == 0) return GDN_OK;
    const void* ptrs[] = {a->src_slots, a->dst_slots};
    for (const void* p : ptrs)
        if (p == nullptr) return fail(GDN_E_INVALID, "gdn_prefill_chunked: NULL slot table");
    if (a->total_tokens > 0) {
        const void* tp[] = {a->q, a->k, a->v, a->g, a->beta, a->o};
        for (const void* p : tp)
            if (p == nullptr) return fail(GDN_E_INVALID, "gdn_prefill_chunked: NULL device pointer");
    }
    const void* vec[] = {a->q, a->k, a->v, a->o};
    for (const void* p : vec)
        if (!aligned(p, 16)) return fail(GDN_E_INVALID, "gdn_prefill_chunked: q, k, v, o must be 16-byte aligned");
    const void* word[] = {a->g, a->beta, a->src_slots, a->dst_slots, a->err_flag, a->cu_seqlens, a->ckpt_slots};
    for (const void* p : word)
        if (!aligned(p, 4)) return fail(GDN_E_INVALID, "gdn_prefill_chunked: g, beta, tables, err_flag must be 4-byte aligned");
    if (workspace == nullptr || !aligned(workspace, 256))
        return fail(GDN_E_INVALID, "gdn_prefill_chunked: workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < plan.bytes)
        return fail(GDN_E_INVALID, "gdn_prefill_chunked: workspace too small (need " + std::to_string(plan.bytes) +
                                       " bytes)");
    return gdn::launch_prefill(pool, a, plan, workspace, stream);
}
