"""fp64 CPU oracle of the gated-delta-rule state update, with the slot semantics.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module. It shares no code with
the HIP path, which must never import it.

Sources
-------
* The hybrid model and its linear-attention layers: 24-ai.news (English),
  "PyTorch: TokenSpeed achieves record 580 tokens/s on Qwen3.5-397B-A17B ...",
  section "What is TokenSpeed and how does it differ from vLLM?" -- the model
  mixes full attention with linear-attention layers built on the Gated Delta
  Network (GDN). The pages do not print the recurrence; this library fixes it
  as the gated delta rule, per token and per value head, with S the
  dv x dk state matrix:

      k^ = k / sqrt(|k|^2 + eps)          q~ = q / sqrt(|q|^2 + eps) * scale
      S <- exp(g) * S                      (decay, g <= 0 is a log-decay)
      S <- S + beta * (v - S k^) k^T       (delta write)
      o  = S q~                            (read-out on the updated state)

  The default scale is 1/sqrt(dk).
* Slots, copy-on-write reuse and index indirection: same article, section
  "What are the key optimizations behind the record?" (items "Hybrid prefix
  caching for GDN/Mamba" and "Mamba State Update optimization"), and
  zubnet.ai (Portuguese), "LightSeek TokenSpeed ...", second paragraph: the
  linear-attention state is checkpointed beside the KV pages, cached
  checkpoints are reused without mutation, and requests address state through
  an index table instead of copying it. Here every request names a source slot
  (read) and a destination slot (written); source slots are never modified.

Readings where the pages are silent (each is stated again where it is used)
-----------------------------------------------------------------------------
* Storage orientation: a pool tile holds H = S^T as a row-major dk x dv array,
  so the pool is ``[num_slots][HV][dk][dv]`` fp32. This oracle converts to S on
  load and back to H on store, and computes in the S orientation of the rule.
* Head grouping: value head h reads key/query head floor(h / (HV / HK)).
* A negative source slot means a zero initial state; a negative destination
  slot means the row is padding and is skipped (its outputs stay unwritten,
  returned here as NaN); a zero-length sequence copies the source state (or
  zero) into the destination.

The token loop is the definition. ``chunked_sequence`` restates the same
recurrence in chunk (WY / UT) form; it exists only so the tests can check that
algebra against the token loop, and the HIP path shares no code with it.
"""

from __future__ import annotations

import numpy as np

# Status codes, mirrored (not shared) by the C library's header.
GDN_OK = 0
GDN_E_INVALID = -1
GDN_E_NO_SLOTS = -3
GDN_E_SLOT_STATE = -4
GDN_E_ALIAS = -5


# ---------------------------------------------------------------------------
# exact upcast of bfloat16 bit patterns
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 values, given as uint16 bit patterns, as exact float64.

    A bfloat16 is the high half of an IEEE float32, so placing the 16 bits in
    the top of a 32-bit word gives the float32 of the same value exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# the rule, one token
# ---------------------------------------------------------------------------

def l2_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gated_delta_token(S, q, k, v, g, beta, scale, eps):
    """One token of the gated delta rule for a batch of heads.

    S: [..., dv, dk] state matrices (fp64); q, k: [..., dk]; v: [..., dv];
    g, beta: [...] per head. Returns (S_new, o) with o: [..., dv].

    The steps are taken in the rule's own order: normalise, decay, delta
    write, then read out on the updated state.
    """
    kh = l2_normalize(k, eps)
    qt = l2_normalize(q, eps) * scale
    g = np.asarray(g, dtype=np.float64)[..., None, None]
    beta = np.asarray(beta, dtype=np.float64)[..., None]
    S = np.exp(g) * S                                   # S <- exp(g) S
    Sk = np.einsum("...ij,...j->...i", S, kh)           # S k^   (dv)
    delta = beta * (np.asarray(v, np.float64) - Sk)     # beta (v - S k^)
    S = S + delta[..., :, None] * kh[..., None, :]      # + (.) k^T
    o = np.einsum("...ij,...j->...i", S, qt)            # o = S q~
    return S, o


def _head_map(HK: int, HV: int) -> np.ndarray:
    if HV % HK != 0:
        raise ValueError("HV must be a multiple of HK")
    return np.arange(HV) // (HV // HK)


def recurrent_sequence(H0, q, k, v, g, beta, scale, eps):
    """Run one sequence token by token.

    H0: [HV, dk, dv] initial tiles in storage orientation (H = S^T).
    q, k: [T, HK, dk]; v: [T, HV, dv]; g, beta: [T, HV] (any float dtype;
    promoted to fp64). Returns (o [T, HV, dv] fp64, H_T [HV, dk, dv] fp64).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, HK, _ = q.shape
    HV = v.shape[1]
    hmap = _head_map(HK, HV)
    S = np.transpose(np.asarray(H0, np.float64), (0, 2, 1)).copy()  # S = H^T
    o = np.empty((T, HV, v.shape[2]), np.float64)
    for t in range(T):
        S, o[t] = gated_delta_token(S, q[t, hmap], k[t, hmap], v[t], g[t], beta[t], scale, eps)
    return o, np.transpose(S, (0, 2, 1)).copy()


# ---------------------------------------------------------------------------
# chunk (WY / UT) form of the same recurrence
# ---------------------------------------------------------------------------

def chunked_sequence(H0, q, k, v, g, beta, scale, eps, chunk):
    """The same sequence, advanced chunk by chunk in the WY / UT form.

    Inside a chunk of c tokens with cumulative log-decay gamma_r = sum_{s<=r} g_s
    and H the state at the chunk start (storage orientation, dk x dv):

        A[r,s] = beta_r exp(gamma_r - gamma_s) (k^_r . k^_s)      for s < r
        T      = (I + A)^-1                                       (unit lower triangular)
        W      = T diag(beta exp(gamma)) K^                       (c x dk)
        U'     = T diag(beta) V                                   (c x dv)
        U      = U' - W H                                         (the delta-rule updates u_r)
        P[r,s] = exp(gamma_r - gamma_s) (q~_r . k^_s)             for s <= r
        O      = diag(exp(gamma)) Q~ H + P U
        H_next = exp(gamma_last) H + (diag(exp(gamma_last - gamma)) K^)^T U

    Derivation: unrolling the token rule inside the chunk gives
    H_r = exp(gamma_r) H + sum_{s<=r} exp(gamma_r - gamma_s) k^_s u_s^T with
    u_r = beta_r (v_r - (exp(g_r) H_{r-1})^T k^_r); substituting H_{r-1} gives
    (I + A) U = diag(beta) V - diag(beta exp(gamma)) K^ H. Decay factors are
    always exp of a non-positive difference, never a ratio of products.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, HK, _ = q.shape
    HV = v.shape[1]
    hmap = _head_map(HK, HV)
    H = np.asarray(H0, np.float64).copy()
    o = np.empty((T, HV, v.shape[2]), np.float64)
    kh_all = l2_normalize(k, eps)[:, hmap]            # [T, HV, dk]
    qt_all = l2_normalize(q, eps)[:, hmap] * scale
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        c = t1 - t0
        tri_strict = np.tril(np.ones((c, c), bool), -1)
        tri_incl = np.tril(np.ones((c, c), bool), 0)
        for h in range(HV):
            Kh = kh_all[t0:t1, h]                     # c x dk
            Qt = qt_all[t0:t1, h]                     # c x dk
            V = v[t0:t1, h]                           # c x dv
            b = beta[t0:t1, h]
            gam = np.cumsum(g[t0:t1, h])
            diff = gam[:, None] - gam[None, :]        # gamma_r - gamma_s
            dec = np.exp(np.where(tri_incl, diff, -np.inf))
            A = np.where(tri_strict, b[:, None] * dec * (Kh @ Kh.T), 0.0)
            Tm = np.linalg.solve(np.eye(c) + A, np.eye(c))
            W = Tm @ ((b * np.exp(gam))[:, None] * Kh)
            Up = Tm @ (b[:, None] * V)
            U = Up - W @ H[h]
            P = np.where(tri_incl, dec * (Qt @ Kh.T), 0.0)
            o[t0:t1, h] = np.exp(gam)[:, None] * (Qt @ H[h]) + P @ U
            Kd = np.exp(gam[-1] - gam)[:, None] * Kh
            H[h] = np.exp(gam[-1]) * H[h] + Kd.T @ U
    return o, H


# ---------------------------------------------------------------------------
# slot-addressed prefill and decode over a state pool
# ---------------------------------------------------------------------------

def prefill(pool, cu_seqlens, src, dst, q, k, v, g, beta, scale, eps, *, chunk=None, ckpt=None,
            ckpt_states=None):
    """Varlen prefill over a slot pool, token by token (or chunk form if chunk).

    pool: [num_slots, HV, dk, dv] float32 tiles (H = S^T); never modified.
    cu_seqlens: [N+1] token offsets; src, dst: [N] slot indices.
    q, k: [T, HK, dk]; v: [T, HV, dv]; g, beta: [T, HV].

    Returns (o, new_pool, finals):
      o        [T, HV, dv] fp64, NaN on rows of skipped (dst < 0) sequences;
      new_pool the pool after the update, float32 (RNE from fp64);
      finals   {n: [HV, dk, dv] fp64} unrounded final state per written sequence.
    Every sequence reads its source tile from the pool as it was on entry, so
    an in-place entry (src == dst) and entries sharing one source all see the
    original bytes; slots that are not destinations keep their bytes.

    Periodic checkpoints (the pages' hybrid prefix caching checkpoints the
    linear-attention state beside the KV pages -- 24-ai.news (English), section
    "What are the key optimizations behind the record?", item "Hybrid prefix
    caching for GDN/Mamba"): ckpt is an optional table over the 64-token
    chunks of all written sequences in order (sequence n owns
    ceil(len_n / 64) entries, skipped sequences own theirs too). When
    ckpt[c] >= 0 the state after chunk c -- after token min(64 (j + 1), len)
    of its sequence, j the chunk's index in it -- is stored to slot ckpt[c]
    (after the destinations). If ckpt_states is a dict it receives
    {c: [HV, dk, dv] fp64} for every stored checkpoint.
    """
    pool = np.asarray(pool, np.float32)
    cu = np.asarray(cu_seqlens, np.int64)
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    T = int(cu[-1])
    HV, dk, dv = pool.shape[1:]
    o = np.full((T, HV, dv), np.nan)
    new_pool = pool.copy()
    finals = {}
    stored = {}
    c_first = 0                                   # first chunk of sequence n in the ckpt table
    for n in range(len(src)):
        a, b = int(cu[n]), int(cu[n + 1])
        nchunks = (b - a + 63) // 64
        c0, c_first = c_first, c_first + nchunks
        if dst[n] < 0:
            continue
        if src[n] >= 0:
            H0 = pool[src[n]].astype(np.float64)
        else:
            H0 = np.zeros((HV, dk, dv))
        if b > a:
            run = (lambda H, s, e: recurrent_sequence(H, q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], scale, eps)) \
                if chunk is None else \
                (lambda H, s, e: chunked_sequence(H, q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], scale, eps, chunk))
            if ckpt is None:
                on, Hn = run(H0, a, b)
                o[a:b] = on
            else:
                Hn = H0
                for j in range(nchunks):
                    s_, e_ = a + 64 * j, min(a + 64 * (j + 1), b)
                    o[s_:e_], Hn = run(Hn, s_, e_)
                    if ckpt[c0 + j] >= 0:
                        stored[c0 + j] = Hn.copy()
        else:
            Hn = H0.copy()
        finals[n] = Hn
        new_pool[dst[n]] = Hn.astype(np.float32)
    for c, Hc in stored.items():
        new_pool[ckpt[c]] = Hc.astype(np.float32)
    if ckpt_states is not None:
        ckpt_states.update(stored)
    return o, new_pool, finals


def decode_step(pool, src, dst, q, k, v, g, beta, scale, eps):
    """One decode token per request: the prefill rule with every length 1.

    q, k: [B, HK, dk]; v: [B, HV, dv]; g, beta: [B, HV]. Same return values as
    ``prefill`` with o of shape [B, HV, dv].
    """
    B = len(np.asarray(src))
    cu = np.arange(B + 1)
    return prefill(pool, cu, src, dst, q, k, v, g, beta, scale, eps)


def verify_step(pool, src, dst, lens, q, k, v, g, beta, scale, eps):
    """Speculative-decode verification: K draft tokens per request in order,
    the state after draft token i stored to its own slot.

    The index indirection the pages describe for speculative decoding (zubnet.ai
    (Portuguese), "LightSeek TokenSpeed ...", second paragraph: an index table
    instead of tensor copies) is read here as follows. Request b starts from
    pool[src[b]] (zero if src[b] < 0) and runs its first lens[b] draft tokens
    through the rule, token by token; after token i the state goes to
    dst[b][i] unless that entry is negative. Accepting a draft prefix is then
    the index write "current slot = dst[b][a]", and a rejected suffix costs
    nothing to undo. lens[b] == 0 skips the request; lens None means all K.

    pool: [num_slots, HV, dk, dv] float32, never modified. src: [B];
    dst: [B, K]; q, k: [B, K, HK, dk]; v: [B, K, HV, dv]; g, beta: [B, K, HV].
    Returns (o [B, K, HV, dv] fp64, NaN for tokens not verified;
    new_pool float32; states {(b, i): [HV, dk, dv] fp64} for every stored i).
    Every request reads its source as the pool held it on entry.
    """
    pool = np.asarray(pool, np.float32)
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    B, K = dst.shape
    lens = np.full(B, K, np.int64) if lens is None else np.asarray(lens, np.int64)
    HV, dk, dv = pool.shape[1:]
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    hmap = _head_map(q.shape[2], HV)
    o = np.full((B, K, HV, dv), np.nan)
    new_pool = pool.copy()
    states = {}
    for b in range(B):
        n = int(lens[b])
        if n <= 0:
            continue
        H0 = pool[src[b]].astype(np.float64) if src[b] >= 0 else np.zeros((HV, dk, dv))
        S = np.transpose(H0, (0, 2, 1)).copy()               # S = H^T
        for i in range(n):
            S, o[b, i] = gated_delta_token(S, q[b, i, hmap], k[b, i, hmap], v[b, i], g[b, i], beta[b, i], scale, eps)
            if dst[b, i] >= 0:
                H = np.transpose(S, (0, 2, 1)).copy()
                states[(b, i)] = H
                new_pool[dst[b, i]] = H.astype(np.float32)
    return o, new_pool, states


def state_pack(pool, slots):
    """Gather slot tiles for a state hand-over (24-ai.news, English, section
    "What are the key optimizations behind the record?", item "Prefill-Decode
    disaggregation": the two phases hand their state over). Entry i is the
    tile of slots[i], or a zero state when slots[i] < 0. Returns float32
    [n, HV, dk, dv]; the pool is not modified."""
    pool = np.asarray(pool, np.float32)
    slots = np.asarray(slots, np.int64)
    out = np.zeros((len(slots),) + pool.shape[1:], np.float32)
    for i, s in enumerate(slots):
        if s >= 0:
            out[i] = pool[s]
    return out


def state_unpack(pool, slots, buffer):
    """Scatter a packed buffer back into slots: pool[slots[i]] <- buffer[i],
    skipping negative entries. Returns the new pool (float32 copy)."""
    new_pool = np.asarray(pool, np.float32).copy()
    for i, s in enumerate(np.asarray(slots, np.int64)):
        if s >= 0:
            new_pool[s] = np.asarray(buffer[i], np.float32)
    return new_pool


# ---------------------------------------------------------------------------
# slot bookkeeping model
# ---------------------------------------------------------------------------

class SlotPoolModel:
    """Reference model of the slot pool's host bookkeeping.

    A slot is free at refcount 0. ``alloc`` hands out the lowest free indices
    (a deterministic choice where the pages give none), all or nothing.
    ``cow`` returns the source itself when this caller is its only holder
    (refcount 1), else a fresh slot; it never changes the source's refcount, so
    a checkpoint stays exactly as it was -- the copy-on-write reuse of cached
    states that the TokenSpeed pages describe.
    """

    def __init__(self, num_slots: int):
        if num_slots <= 0:
            raise ValueError("num_slots must be positive")
        self.ref = [0] * num_slots

    @property
    def capacity(self) -> int:
        return len(self.ref)

    def num_free(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def refcount(self, slot: int):
        if not 0 <= slot < len(self.ref):
            return GDN_E_INVALID, None
        return GDN_OK, self.ref[slot]

    def alloc(self, n: int):
        if n < 0:
            return GDN_E_INVALID, []
        free = [i for i, r in enumerate(self.ref) if r == 0]
        if len(free) < n:
            return GDN_E_NO_SLOTS, []
        out = free[:n]
        for s in out:
            self.ref[s] = 1
        return GDN_OK, out

    def retain(self, slot: int):
        if not 0 <= slot < len(self.ref):
            return GDN_E_INVALID
        if self.ref[slot] == 0:
            return GDN_E_SLOT_STATE
        self.ref[slot] += 1
        return GDN_OK

    def release(self, slot: int):
        if not 0 <= slot < len(self.ref):
            return GDN_E_INVALID
        if self.ref[slot] == 0:
            return GDN_E_SLOT_STATE
        self.ref[slot] -= 1
        return GDN_OK

    def cow(self, src: int):
        if src >= len(self.ref):
            return GDN_E_INVALID, -1
        if src >= 0 and self.ref[src] == 0:
            return GDN_E_SLOT_STATE, -1
        if src >= 0 and self.ref[src] == 1:
            return GDN_OK, src
        st, out = self.alloc(1)
        if st != GDN_OK:
            return st, -1
        return GDN_OK, out[0]

    def validate(self, src, dst):
        """Range, allocation and aliasing checks of a src/dst slot table.

        Pass 1, entry by entry: a slot index >= capacity is GDN_E_INVALID; a
        non-negative slot that is not allocated is GDN_E_SLOT_STATE (src is
        checked before dst). Pass 2: two entries with the same destination, or
        a destination equal to another entry's source, is GDN_E_ALIAS. A
        source shared by several entries, and src == dst within one entry, are
        allowed. Negative indices mean "none" and are never checked further.
        """
        src = list(src)
        dst = list(dst)
        if len(src) != len(dst):
            return GDN_E_INVALID
        cap = len(self.ref)
        for s, d in zip(src, dst):
            for x in (s, d):
                if x >= cap:
                    return GDN_E_INVALID
                if x >= 0 and self.ref[x] == 0:
                    return GDN_E_SLOT_STATE
        seen = set()
        for d in dst:
            if d >= 0:
                if d in seen:
                    return GDN_E_ALIAS
                seen.add(d)
        for i, d in enumerate(dst):
            if d < 0:
                continue
            for j, s in enumerate(src):
                if j != i and s == d:
                    return GDN_E_ALIAS
        return GDN_OK


class PrefixCacheModel:
    """Reference model of the logical prefix cache (the pages' C++ layer of
    hybrid prefix caching with radix-tree matching over linear-attention
    state slots: 24-ai.news (English), section "What are the key
    optimizations behind the record?", item "Hybrid prefix caching for
    GDN/Mamba"). A plain dict from token prefix to [slot, stamp] over a
    SlotPoolModel: the tree only makes the same answers fast.

    insert: the prefix gets the slot (the cache retains it) unless it already
    has one. match: the longest stored prefix of the tokens; a hit retains
    its slot for the caller and restamps it. evict: drop the checkpoints whose
    slot only the cache holds (refcount 1), oldest stamp first, until the pool
    has `want_free` free slots. Stamps come from one clock advanced by every
    insert and every hit.
    """

    def __init__(self, pool_model):
        self.pool = pool_model
        self.entries = {}
        self.clock = 0

    def insert(self, tokens, slot):
        key = tuple(int(t) for t in tokens)
        if len(key) == 0 or slot < 0 or slot >= self.pool.capacity:
            return GDN_E_INVALID, 0
        if self.pool.refcount(slot)[1] == 0:
            return GDN_E_SLOT_STATE, 0
        if key in self.entries:
            return GDN_OK, 0
        self.pool.retain(slot)
        self.clock += 1
        self.entries[key] = [slot, self.clock]
        return GDN_OK, 1

    def match(self, tokens):
        toks = tuple(int(t) for t in tokens)
        best = None
        for key in self.entries:
            if len(key) <= len(toks) and toks[:len(key)] == key and (best is None or len(key) > len(best)):
                best = key
        if best is None:
            return GDN_OK, 0, -1
        slot = self.entries[best][0]
        self.pool.retain(slot)
        self.clock += 1
        self.entries[best][1] = self.clock
        return GDN_OK, len(best), slot

    def evict(self, want_free):
        dropped = 0
        for key in sorted(self.entries, key=lambda k: self.entries[k][1]):
            if self.pool.num_free() >= want_free:
                break
            slot = self.entries[key][0]
            if self.pool.refcount(slot)[1] != 1:
                continue
            self.pool.release(slot)
            del self.entries[key]
            dropped += 1
        return GDN_OK, dropped

    def size(self):
        return len(self.entries)
