/*
 * gdn.h -- C ABI of libgdn.so: the recurrent-state update of Gated Delta
 * Network (GDN) linear-attention layers on AMD MI355X (gfx950).
 *
 * The operation. The TokenSpeed article (24-ai.news, English, "PyTorch:
 * TokenSpeed achieves record 580 tokens/s on Qwen3.5-397B-A17B ...", section
 * "What is TokenSpeed and how does it differ from vLLM?") names linear-attention
 * layers built on the Gated Delta Network inside a hybrid model; the pages do
 * not print the recurrence. This library implements the gated delta rule, per
 * token and per value head, with S the dv x dk state matrix:
 *
 *     k^ = k / sqrt(|k|^2 + l2_eps)        q~ = q / sqrt(|q|^2 + l2_eps) * scale
 *     S  <- exp(g) S
 *     S  <- S + beta (v - S k^) k^T
 *     o   = S q~
 *
 * Slots and index indirection. Same article, section "What are the key
 * optimizations behind the record?", items "Hybrid prefix caching for
 * GDN/Mamba" (state reuse under copy-on-write) and "Mamba State Update
 * optimization" (index indirection in place of copying state between steps);
 * zubnet.ai (Portuguese), "LightSeek TokenSpeed ...", second paragraph (the
 * linear-attention state is checkpointed beside the KV pages and cached
 * checkpoints are reused without mutation). Here states live in a pool of
 * fixed-size slots; every request names a source slot that is only read and a
 * destination slot that is written, so advancing a request is an index write
 * and a cached checkpoint is never modified.
 *
 * Storage. A pool is caller-owned device memory of
 *     num_slots * HV * dk * dv  float32,  layout [slot][HV][dk][dv],
 * each (slot, head) tile holding H = S^T row-major (dk rows of dv floats).
 * q and k are [tokens][HK][dk]; v and o are [tokens][HV][dv]; g and beta are
 * float32 [tokens][HV]. Value head h reads key/query head h / (HV / HK).
 *
 * Conventions shared by every call:
 *   - Return value: GDN_OK (0) or a negative GDN_E_* code. A failing call
 *     changes no state; gdn_last_error() then returns a message (thread-local,
 *     valid until the next failing call on the same thread).
 *   - Device pointers are HIP device addresses; "stream" is a hipStream_t
 *     passed as void* (NULL = the default stream). Launching calls are
 *     asynchronous: they enqueue work on the stream, never synchronise the
 *     host, never allocate, and may be captured into a HIP graph.
 *   - Pool bookkeeping calls are host-only and touch no device memory. They
 *     are not thread-safe; one scheduler thread serialises them.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define GDN_OK             0
#define GDN_E_INVALID     -1  /* null pointer, bad size, bad alignment, index out of range */
#define GDN_E_UNSUPPORTED -2  /* a dtype / head-size combination this build has no kernel for */
#define GDN_E_NO_SLOTS    -3  /* not enough free slots; nothing was allocated */
#define GDN_E_SLOT_STATE  -4  /* slot is free where an allocated slot is required */
#define GDN_E_ALIAS       -5  /* a destination is repeated or is another entry's source */
#define GDN_E_HIP         -6  /* the HIP runtime reported an error (message copied) */

/* element types of q, k, v and o (g, beta and the pool are always float32) */
#define GDN_DTYPE_F32  0
#define GDN_DTYPE_BF16 1

/* bits of the optional device error flag (int32, OR-ed in by kernels; only the
 * end of a decode-graph replay clears it) */
#define GDN_ERRFLAG_SLOT_RANGE 1   /* a src/dst slot index >= num_slots was skipped */
#define GDN_ERRFLAG_DRAFT_LEN  2   /* a draft length outside [0, num_draft] was skipped (verify) */

typedef struct gdn_pool gdn_pool;   /* opaque host-side handle */

/* ------------------------------------------------------------------------ */
/* slot pool (host bookkeeping over caller-owned device storage)             */
/* ------------------------------------------------------------------------ */

/* Create a pool handle over `storage` (device, caller-owned, >= 16-byte
 * aligned, num_slots*num_v_heads*dk*dv floats). The pool never frees or reads
 * the storage itself; all slots start free (refcount 0).
 * dk, dv must be in {16, 32, 64, 128}. Errors: GDN_E_INVALID. */
int gdn_state_pool_create(int32_t num_slots, int32_t num_v_heads, int32_t dk, int32_t dv,
                          float* storage, gdn_pool** out);

/* Free the host bookkeeping (not the storage). NULL is accepted. */
int gdn_state_pool_destroy(gdn_pool* pool);

/* Allocate n slots, lowest free indices first, each with refcount 1, written
 * to out[0..n-1] (host). All or nothing: GDN_E_NO_SLOTS leaves the pool
 * unchanged. n < 0 or out == NULL with n > 0: GDN_E_INVALID. */
int gdn_state_pool_alloc(gdn_pool* pool, int32_t n, int32_t* out);

/* refcount += 1 / -= 1 (the slot becomes free at 0). Out of range:
 * GDN_E_INVALID; slot free: GDN_E_SLOT_STATE. */
int gdn_state_pool_retain(gdn_pool* pool, int32_t slot);
int gdn_state_pool_release(gdn_pool* pool, int32_t slot);

/* Copy-on-write target for a caller about to advance state read from `src`:
 * if src >= 0 and refcount(src) == 1 the caller is its only holder and *dst =
 * src (update in place); if src < 0 (no state) or refcount(src) > 1 a fresh
 * slot is allocated (refcount 1). The refcount of src is never changed and no
 * state bytes move: the O(1) pointer update of the pages. Errors:
 * GDN_E_INVALID (src >= num_slots, dst NULL), GDN_E_SLOT_STATE (src free),
 * GDN_E_NO_SLOTS. */
int gdn_state_pool_cow(gdn_pool* pool, int32_t src, int32_t* dst);

/* Check a slot table (host copies of what the kernels will read).
 * Pass 1, entry by entry (src before dst): index >= num_slots ->
 * GDN_E_INVALID; non-negative index of a free slot -> GDN_E_SLOT_STATE.
 * Pass 2: a destination used twice, or equal to a different entry's source ->
 * GDN_E_ALIAS. A source shared by several entries, src == dst in one entry
 * (in place) and negative indices (none) are allowed. Kernels assume a table
 * that passed this check and do not re-check aliasing. */
int gdn_state_pool_validate(const gdn_pool* pool, int32_t n, const int32_t* src_host,
                            const int32_t* dst_host);

/* queries */
int gdn_state_pool_refcount(const gdn_pool* pool, int32_t slot, int32_t* out);
int gdn_state_pool_num_free(const gdn_pool* pool, int32_t* out);
int gdn_state_pool_capacity(const gdn_pool* pool, int32_t* out);

/* ------------------------------------------------------------------------ */
/* prefix cache: the logical layer over slot checkpoints                     */
/* ------------------------------------------------------------------------ */

/* 24-ai.news (English), section "What are the key optimizations behind the
 * record?", item "Hybrid prefix caching for GDN/Mamba": context caching is
 * split between a C++ logical cache and the physical tensors, with radix-tree
 * matching extended to the linear-attention state slots and copy-on-write
 * reuse. This is that logical layer for one pool: a radix tree over token ids
 * whose nodes own slot checkpoints (a slot holding the state after exactly
 * that prefix, written e.g. by a prefill checkpoint). The cache holds one
 * reference (refcount) on every slot it owns; callers keep their own. Not
 * thread-safe, like the pool. Errors: GDN_E_INVALID (NULL, n <= 0, slot out
 * of range), GDN_E_SLOT_STATE (a free slot), GDN_E_NO_SLOTS (create: none). */
typedef struct gdn_prefix_cache gdn_prefix_cache;

/* A cache over `pool`, which must outlive it. */
int gdn_prefix_cache_create(gdn_pool* pool, gdn_prefix_cache** out);
/* Releases every checkpoint's reference, then frees the cache. NULL is a no-op. */
int gdn_prefix_cache_destroy(gdn_prefix_cache* cache);
/* Record that allocated `slot` holds the state after tokens[0..n). The cache
 * retains it (*inserted = 1). If that prefix already has a checkpoint nothing
 * changes (*inserted = 0; the caller keeps its own reference either way). */
int gdn_prefix_cache_insert(gdn_prefix_cache* cache, const int32_t* tokens, int32_t n, int32_t slot,
                            int32_t* inserted);
/* Longest prefix of tokens[0..n) that has a checkpoint: *len tokens in slot
 * *slot, retained once more for the caller (who releases it when done) and
 * marked most recently used; *len = 0 and *slot = -1 on a miss. A request
 * resumes from it copy-on-write: read the slot as its source, write elsewhere. */
int gdn_prefix_cache_match(gdn_prefix_cache* cache, const int32_t* tokens, int32_t n, int32_t* len, int32_t* slot);
/* Drop checkpoints whose slot the cache alone holds (refcount 1), least
 * recently inserted or matched first, until the pool has at least
 * `want_free` free slots or no such checkpoint is left. *dropped = how many. */
int gdn_prefix_cache_evict(gdn_prefix_cache* cache, int32_t want_free, int32_t* dropped);
/* Number of checkpoints held. */
int gdn_prefix_cache_size(const gdn_prefix_cache* cache, int32_t* out);

/* ------------------------------------------------------------------------ */
/* state transfer                                                            */
/* ------------------------------------------------------------------------ */

/* 24-ai.news (English), section "What are the key optimizations behind the
 * record?", item "Prefill-Decode disaggregation": the context-filling and
 * token-generation phases run apart and hand their state over. These two calls
 * are the one-GPU half of that hand-over. pack copies the tiles of n slots into
 * one contiguous device buffer that a transport can move; unpack writes such a
 * buffer into slots of a pool with the same head shape (HV, dk, dv).
 *
 * slots: [n] device int32. buffer: [n][HV][dk][dv] device float32, 16-byte
 * aligned. pack: entry i <- pool[slots[i]]; slots[i] < 0 writes a zero state.
 * unpack: pool[slots[i]] <- entry i; slots[i] < 0 skips the entry; the
 * non-negative slots must be distinct. A slot >= num_slots skips its entry and
 * sets GDN_ERRFLAG_SLOT_RANGE in err_flag (optional). Bit-exact copies, no
 * refcount change (the caller owns the bookkeeping). Asynchronous on `stream`,
 * no allocation, graph-capturable. Errors: GDN_E_INVALID (n < 0, NULL or
 * misaligned pointers when n > 0). */
int gdn_state_pool_pack(const gdn_pool* pool, int32_t n, const int32_t* slots, float* buffer, int32_t* err_flag,
                        void* stream);
int gdn_state_pool_unpack(const gdn_pool* pool, int32_t n, const int32_t* slots, const float* buffer,
                          int32_t* err_flag, void* stream);

/* ------------------------------------------------------------------------ */
/* decode: one token per request                                             */
/* ------------------------------------------------------------------------ */

typedef struct gdn_decode_args {
    int32_t batch;          /* B >= 0 requests */
    int32_t num_k_heads;    /* HK, divides num_v_heads */
    int32_t num_v_heads;    /* HV, must equal the pool's */
    int32_t dk, dv;         /* must equal the pool's */
    int32_t dtype;          /* GDN_DTYPE_F32 or GDN_DTYPE_BF16: q, k, v, o */
    const void* q;          /* [B][HK][dk] device */
    const void* k;          /* [B][HK][dk] device */
    const void* v;          /* [B][HV][dv] device */
    const float* g;         /* [B][HV] device, log-decay (<= 0 expected) */
    const float* beta;      /* [B][HV] device */
    void* o;                /* [B][HV][dv] device, written for rows with dst >= 0 */
    const int32_t* src_slots;  /* [B] device: < 0 = zero initial state */
    const int32_t* dst_slots;  /* [B] device: < 0 = padding row, skipped */
    float scale;            /* applied to q after normalisation (usually dk^-1/2) */
    float l2_eps;           /* epsilon of the q/k L2 normalisation */
    int32_t* err_flag;      /* optional device int32; GDN_ERRFLAG_* bits OR-ed in */
} gdn_decode_args;

/* Advance every request by one token: o[b] = read-out after the update;
 * pool[dst[b]] = updated state; pool[src[b]] untouched unless src == dst.
 * All device pointers >= 16-byte aligned. Slot indices >= num_slots are
 * skipped in the kernel and flagged in err_flag. Asynchronous on `stream`,
 * no allocation, no host synchronisation, graph-capturable. */
int gdn_decode_step(const gdn_pool* pool, const gdn_decode_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* speculative-decode verification: K draft tokens per request               */
/* ------------------------------------------------------------------------ */

/* zubnet.ai (Portuguese), "LightSeek TokenSpeed ...", second paragraph: during
 * speculative decoding the engine addresses state through an index table
 * instead of copying tensors. Here one launch runs each request's draft
 * tokens through the rule in order and stores the state after draft token i
 * to its own slot, so accepting a draft prefix is the index write
 * "current slot = dst[b][a]" and a rejected suffix needs no undo. */
typedef struct gdn_verify_args {
    int32_t batch;          /* B >= 0 requests */
    int32_t num_draft;      /* K, 1 <= K <= 64 draft tokens per request */
    int32_t num_k_heads;    /* HK, divides num_v_heads */
    int32_t num_v_heads;    /* HV, must equal the pool's */
    int32_t dk, dv;         /* must equal the pool's */
    int32_t dtype;          /* GDN_DTYPE_F32 or GDN_DTYPE_BF16: q, k, v, o */
    const void* q;          /* [B][K][HK][dk] device */
    const void* k;          /* [B][K][HK][dk] device */
    const void* v;          /* [B][K][HV][dv] device */
    const float* g;         /* [B][K][HV] device, log-decay */
    const float* beta;      /* [B][K][HV] device */
    void* o;                /* [B][K][HV][dv] device, written for verified tokens */
    const int32_t* src_slots;  /* [B] device: < 0 = zero initial state */
    const int32_t* dst_slots;  /* [B][K] device: state after draft token i -> dst[b*K+i]; < 0 = not stored */
    const int32_t* draft_lens; /* [B] device, or NULL for all K: request b verifies its first
                                  draft_lens[b] tokens (0 = request skipped) */
    float scale;            /* applied to q after normalisation (usually dk^-1/2) */
    float l2_eps;
    int32_t* err_flag;      /* optional device int32; GDN_ERRFLAG_* bits OR-ed in */
} gdn_verify_args;

/* For every request, read pool[src[b]] once, apply its verified draft tokens
 * one after another (each exactly as gdn_decode_step would), write the output
 * of every verified token and store the state after token i to dst[b][i]
 * when that entry is >= 0. Tokens past draft_lens[b] leave outputs and slots
 * untouched. Slot tables follow gdn_state_pool_validate applied to the flat
 * table of pairs (src[b], dst[b][i]): destinations distinct, none equal to
 * another request's source; dst[b][i] == src[b] (in place) is allowed. A
 * request with an out-of-range slot or draft length is skipped and flagged in
 * err_flag. Asynchronous on `stream`, no allocation, no host synchronisation,
 * graph-capturable. */
int gdn_decode_verify(const gdn_pool* pool, const gdn_verify_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* recorded decode step: a whole step of decode launches as one HIP graph    */
/* ------------------------------------------------------------------------ */

/* The TokenSpeed article (24-ai.news, English, section "What are the key
 * optimizations behind the record?", item "CUDA graph recording") records the
 * whole decode loop as one graph so that kernels are not launched one by one;
 * zubnet.ai (Portuguese), second paragraph, adds the overlap of host and GPU
 * work around it: graph capture, asynchronous host-to-device copies from
 * pinned memory, layer barriers built on events, and sentinels written by the
 * GPU so the host need not read device memory back. Here:
 *   - a list of decode launches ("entries", e.g. one per GDN layer of a model,
 *     or several steps of one layer) is recorded once and replayed per step;
 *   - the slot tables stay in device memory: every entry reads the src/dst
 *     tables its args name, which the caller (or GPU code, e.g. an acceptance
 *     kernel) rewrites between replays in stream order, typically by an
 *     asynchronous copy from pinned host memory;
 *   - each replay ends with a sentinel kernel that reads the shared err_flag,
 *     clears it, counts the replay and writes (count, flags) into pinned host
 *     memory, which gdn_decode_graph_poll reads without any GPU call;
 *   - with GDN_GRAPH_LAYER_EVENTS an event is recorded after every entry, and
 *     a stream or the host can wait for entry i of the latest replay alone. */

typedef struct gdn_decode_graph gdn_decode_graph;   /* opaque */

#define GDN_GRAPH_LAYER_EVENTS 1   /* record an event after every entry */
#define GDN_GRAPH_MAX_ENTRIES 4096

/* Record `num_entries` decode launches, in order, into a graph. entries[i] is
 * checked as by gdn_decode_step and must have batch >= 1; every entry must
 * name the same non-NULL err_flag. storages (optional, NULL = all entries use
 * the pool's storage) gives entry i's slot storage: NULL for the pool's own,
 * else device memory of the pool's shape [num_slots][HV][dk][dv] float32,
 * 16-byte aligned (one GDN layer's states; all layers share the pool's slot
 * numbering). Every pointer is baked into the graph: the buffers must outlive
 * it, and their contents are read at each replay. flags: 0 or
 * GDN_GRAPH_LAYER_EVENTS. The library allocates the graph, its events, a
 * device word and a pinned host word; nothing is enqueued on caller streams.
 * On failure nothing is left allocated and *out is unchanged. */
int gdn_decode_graph_create(const gdn_pool* pool, int32_t num_entries, const gdn_decode_args* entries,
                            float* const* storages, int32_t flags, gdn_decode_graph** out);

/* Enqueue one replay on `stream`. Replays of one graph must not overlap:
 * launch them on one stream, or order them. Asynchronous, no allocation. */
int gdn_decode_graph_launch(gdn_decode_graph* graph, void* stream);

/* Replays finished so far (the sentinel count, 0 before the first) and the
 * err_flag bits the last of them saw. Host memory only: no GPU call, no
 * synchronisation. A count behind the number of launches means a replay is
 * still running. */
int gdn_decode_graph_poll(const gdn_decode_graph* graph, uint32_t* replays, int32_t* flags);

/* Make `stream` wait, on the GPU, until entry `entry` of the latest enqueued
 * replay has finished (needs GDN_GRAPH_LAYER_EVENTS). */
int gdn_decode_graph_wait_entry(const gdn_decode_graph* graph, int32_t entry, void* stream);

/* Block the host until entry `entry` of the latest enqueued replay has
 * finished (needs GDN_GRAPH_LAYER_EVENTS). */
int gdn_decode_graph_sync_entry(const gdn_decode_graph* graph, int32_t entry);

/* Wait for the device to go idle, then free the graph and everything the
 * library allocated for it. NULL is a no-op. */
int gdn_decode_graph_destroy(gdn_decode_graph* graph);

/* ------------------------------------------------------------------------ */
/* chunked prefill: variable-length sequences packed by cu_seqlens           */
/* ------------------------------------------------------------------------ */

typedef struct gdn_prefill_args {
    int32_t num_seqs;             /* N >= 0 */
    int32_t total_tokens;         /* T = cu_seqlens[N] */
    const int32_t* cu_seqlens;    /* [N+1] device, 0 = cu[0] <= cu[1] <= ... */
    const int32_t* cu_seqlens_host; /* [N+1] host mirror, equal to cu_seqlens: grid sizing,
                                     checks, and for N <= 32 the first chunk of every
                                     sequence, passed to the kernels by value */
    int32_t chunk_size;           /* must be 64 */
    int32_t num_k_heads, num_v_heads, dk, dv;
    int32_t dtype;                /* GDN_DTYPE_BF16: chunked form on bf16 matrix cores;
                                     GDN_DTYPE_F32: the same chunked form with every product
                                     on fp32 matrix cores, for fp32 accuracy (never split
                                     into segments); dk, dv in {16, 32, 64, 128} for both */
    const void* q;                /* [T][HK][dk] device */
    const void* k;                /* [T][HK][dk] device */
    const void* v;                /* [T][HV][dv] device */
    const float* g;               /* [T][HV] device */
    const float* beta;            /* [T][HV] device */
    void* o;                      /* [T][HV][dv] device */
    const int32_t* src_slots;     /* [N] device: < 0 = zero initial state */
    const int32_t* dst_slots;     /* [N] device: < 0 = sequence skipped */
    float scale;
    float l2_eps;
    int32_t* err_flag;            /* optional, as for decode */
    const int32_t* ckpt_slots;    /* optional [C] device, C = sum over sequences of ceil(len / 64)
                                     (sequence order, skipped sequences included): when
                                     ckpt_slots[c] >= 0 the state after chunk c is also stored
                                     to that slot (NULL: no checkpoints) */
} gdn_prefill_args;

/* Bytes of device workspace gdn_prefill_chunked needs for these args (depends
 * on N, the chunk count from cu_seqlens_host, the head shape and the dtype:
 * per (chunk, value head) the T and P matrices, 16 KiB in bf16 or 20 KiB as
 * fp32 blocks, and 1.25 KiB of scale rows; plus, for bf16 calls the planner
 * splits, per-segment end states and transitions). */
int gdn_prefill_workspace_bytes(const gdn_pool* pool, const gdn_prefill_args* args, size_t* bytes);

/* Run every sequence through the rule from its source state and write the
 * final state to its destination slot. With ckpt_slots the states at the
 * chosen 64-token chunk boundaries are stored as well: the periodic
 * checkpoints of the pages' hybrid prefix caching, which keeps the
 * linear-attention state beside the KV pages (24-ai.news, English, section
 * "What are the key optimizations behind the record?", item "Hybrid prefix
 * caching for GDN/Mamba"). Checkpoint slots must be distinct and differ from
 * every source and destination of the call; an out-of-range one is skipped
 * and flagged. Chunks of 64 tokens restart at every
 * sequence boundary; a zero-length sequence copies the source state (zero if
 * src < 0) to the destination. `workspace` is caller-owned device memory of
 * at least gdn_prefill_workspace_bytes, 256-byte aligned; its contents are
 * scratch. Asynchronous on `stream`, no allocation, no host sync. */
int gdn_prefill_chunked(const gdn_pool* pool, const gdn_prefill_args* args, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The same prefill for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Identical arguments and results to gdn_prefill_chunked, but the
 * workspace is a file-scope device array inside the library, one per GPU,
 * GDN_PREFILL_STATIC_WORKSPACE_BYTES (64 MiB) long, held until the process
 * ends. The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); on its first use on a GPU it looks up that GPU's copy of
 * the array once. A call whose workspace (gdn_prefill_workspace_bytes)
 * exceeds the array returns GDN_E_INVALID and enqueues nothing: 64 MiB covers
 * one 4096-token call at 16 key / 32 value heads of 128 x 128 in either
 * dtype (bf16 52.5 MiB, fp32 42.5 MiB). The workspace needs no clearing
 * between calls. Every call on one GPU shares that GPU's array: two calls
 * whose work overlaps on one GPU (different streams, or graphs replayed
 * concurrently) race on it and must be serialised by the caller. The device
 * is the stream's (the current device for the NULL stream). */
#define GDN_PREFILL_STATIC_WORKSPACE_BYTES (64u << 20)
int gdn_prefill_chunked_static(const gdn_pool* pool, const gdn_prefill_args* args, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
