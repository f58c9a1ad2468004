"""Thin ctypes binding over libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream; every step of the state update runs in the library's
HIP kernels. If the library has not been built this module raises on first use
-- there is no fallback path.

Names follow the C ABI: ``gdn_state_pool_*``, ``gdn_decode_step``,
``gdn_prefill_workspace_bytes``, ``gdn_prefill_chunked``, ``gdn_last_error``.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int32, c_size_t, c_void_p

import numpy as np

GDN_OK = 0
GDN_E_INVALID = -1
GDN_E_UNSUPPORTED = -2
GDN_E_NO_SLOTS = -3
GDN_E_SLOT_STATE = -4
GDN_E_ALIAS = -5
GDN_E_HIP = -6

GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

GDN_ERRFLAG_SLOT_RANGE = 1
GDN_ERRFLAG_DRAFT_LEN = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

EXPORTED = (
    "gdn_state_pool_create", "gdn_state_pool_destroy", "gdn_state_pool_alloc",
    "gdn_state_pool_retain", "gdn_state_pool_release", "gdn_state_pool_cow",
    "gdn_state_pool_validate", "gdn_state_pool_refcount", "gdn_state_pool_num_free",
    "gdn_state_pool_capacity", "gdn_decode_step", "gdn_prefill_workspace_bytes",
    "gdn_decode_verify", "gdn_prefill_chunked", "gdn_last_error", "gdn_state_pool_pack",
    "gdn_state_pool_unpack", "gdn_prefix_cache_create", "gdn_prefix_cache_destroy", "gdn_prefix_cache_insert",
    "gdn_prefix_cache_match", "gdn_prefix_cache_evict", "gdn_prefix_cache_size",
    "gdn_decode_graph_create", "gdn_decode_graph_launch", "gdn_decode_graph_poll",
    "gdn_decode_graph_wait_entry", "gdn_decode_graph_sync_entry", "gdn_decode_graph_destroy",
    "gdn_prefill_chunked_static",
)

GDN_PREFILL_STATIC_WORKSPACE_BYTES = 64 << 20

GDN_GRAPH_LAYER_EVENTS = 1
GDN_GRAPH_MAX_ENTRIES = 4096


class GdnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("num_k_heads", c_int32), ("num_v_heads", c_int32),
        ("dk", c_int32), ("dv", c_int32), ("dtype", c_int32),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("g", c_void_p), ("beta", c_void_p),
        ("o", c_void_p), ("src_slots", c_void_p), ("dst_slots", c_void_p),
        ("scale", c_float), ("l2_eps", c_float), ("err_flag", c_void_p),
    ]


class VerifyArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("num_draft", c_int32), ("num_k_heads", c_int32), ("num_v_heads", c_int32),
        ("dk", c_int32), ("dv", c_int32), ("dtype", c_int32),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("g", c_void_p), ("beta", c_void_p),
        ("o", c_void_p), ("src_slots", c_void_p), ("dst_slots", c_void_p), ("draft_lens", c_void_p),
        ("scale", c_float), ("l2_eps", c_float), ("err_flag", c_void_p),
    ]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", c_int32), ("total_tokens", c_int32),
        ("cu_seqlens", c_void_p), ("cu_seqlens_host", c_void_p),
        ("chunk_size", c_int32), ("num_k_heads", c_int32), ("num_v_heads", c_int32),
        ("dk", c_int32), ("dv", c_int32), ("dtype", c_int32),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("g", c_void_p), ("beta", c_void_p),
        ("o", c_void_p), ("src_slots", c_void_p), ("dst_slots", c_void_p),
        ("scale", c_float), ("l2_eps", c_float), ("err_flag", c_void_p), ("ckpt_slots", c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn.so once and declare its signatures. Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libgdn.so not found at {path}; build it first "
            "(python -m hybrid_linear_attention_02_amd.build or __graft_entry__.build())")
    # One HIP runtime per process: torch carries its own libamdhip64 (soname
    # libamdhip64.so.7, which its libraries request by file name), and
    # libgdn.so binds to whichever libamdhip64.so.7 is loaded first. Loading
    # torch first makes the library use torch's runtime, so the tensors,
    # streams and graphs torch hands over are that runtime's own. Opened the
    # other way round, the process would hold two runtimes.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = c_void_p
    sig = {
        "gdn_state_pool_create": ([c_int32, c_int32, c_int32, c_int32, P, POINTER(P)], c_int32),
        "gdn_state_pool_destroy": ([P], c_int32),
        "gdn_state_pool_alloc": ([P, c_int32, POINTER(c_int32)], c_int32),
        "gdn_state_pool_retain": ([P, c_int32], c_int32),
        "gdn_state_pool_release": ([P, c_int32], c_int32),
        "gdn_state_pool_cow": ([P, c_int32, POINTER(c_int32)], c_int32),
        "gdn_state_pool_validate": ([P, c_int32, POINTER(c_int32), POINTER(c_int32)], c_int32),
        "gdn_state_pool_refcount": ([P, c_int32, POINTER(c_int32)], c_int32),
        "gdn_state_pool_num_free": ([P, POINTER(c_int32)], c_int32),
        "gdn_state_pool_capacity": ([P, POINTER(c_int32)], c_int32),
        "gdn_prefix_cache_create": ([P, POINTER(P)], c_int32),
        "gdn_prefix_cache_destroy": ([P], c_int32),
        "gdn_prefix_cache_insert": ([P, POINTER(c_int32), c_int32, c_int32, POINTER(c_int32)], c_int32),
        "gdn_prefix_cache_match": ([P, POINTER(c_int32), c_int32, POINTER(c_int32), POINTER(c_int32)], c_int32),
        "gdn_prefix_cache_evict": ([P, c_int32, POINTER(c_int32)], c_int32),
        "gdn_prefix_cache_size": ([P, POINTER(c_int32)], c_int32),
        "gdn_state_pool_pack": ([P, c_int32, P, P, P, P], c_int32),
        "gdn_state_pool_unpack": ([P, c_int32, P, P, P, P], c_int32),
        "gdn_decode_step": ([P, POINTER(DecodeArgs), P], c_int32),
        "gdn_decode_verify": ([P, POINTER(VerifyArgs), P], c_int32),
        "gdn_prefill_workspace_bytes": ([P, POINTER(PrefillArgs), POINTER(c_size_t)], c_int32),
        "gdn_prefill_chunked": ([P, POINTER(PrefillArgs), P, c_size_t, P], c_int32),
        "gdn_prefill_chunked_static": ([P, POINTER(PrefillArgs), P], c_int32),
        "gdn_decode_graph_create": ([P, c_int32, POINTER(DecodeArgs), POINTER(P), c_int32, POINTER(P)], c_int32),
        "gdn_decode_graph_launch": ([P, P], c_int32),
        "gdn_decode_graph_poll": ([P, POINTER(ctypes.c_uint32), POINTER(c_int32)], c_int32),
        "gdn_decode_graph_wait_entry": ([P, c_int32, P], c_int32),
        "gdn_decode_graph_sync_entry": ([P, c_int32], c_int32),
        "gdn_decode_graph_destroy": ([P], c_int32),
        "gdn_last_error": ([], c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def gdn_last_error() -> str:
    return load_library().gdn_last_error().decode()


def _check(status: int) -> None:
    if status != GDN_OK:
        raise GdnError(status, gdn_last_error())


# ---------------------------------------------------------------------------
# slot pool
# ---------------------------------------------------------------------------

class StatePool:
    """A pool handle plus the device tensor that holds its slots.

    ``storage`` is float32 [num_slots, HV, dk, dv] (each tile is H = S^T, dk
    rows of dv). The tensor is owned here (or by the caller if passed in); the
    C handle only keeps its address.
    """

    def __init__(self, handle: int, storage, num_slots: int, num_v_heads: int, dk: int, dv: int):
        self.handle = handle
        self.storage = storage
        self.num_slots, self.num_v_heads, self.dk, self.dv = num_slots, num_v_heads, dk, dv

    def close(self) -> None:
        if self.handle:
            load_library().gdn_state_pool_destroy(c_void_p(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # convenience methods, each one ABI call
    def alloc(self, n: int):
        return gdn_state_pool_alloc(self, n)

    def retain(self, slot: int) -> None:
        gdn_state_pool_retain(self, slot)

    def release(self, slot: int) -> None:
        gdn_state_pool_release(self, slot)

    def cow(self, src: int) -> int:
        return gdn_state_pool_cow(self, src)

    def validate(self, src, dst) -> None:
        gdn_state_pool_validate(self, src, dst)

    def refcount(self, slot: int) -> int:
        return gdn_state_pool_refcount(self, slot)

    def num_free(self) -> int:
        return gdn_state_pool_num_free(self)

    def capacity(self) -> int:
        return gdn_state_pool_capacity(self)


def gdn_state_pool_create(num_slots: int, num_v_heads: int, dk: int, dv: int, storage=None,
                          device: str = "cuda") -> StatePool:
    """Create a pool over ``storage`` (a float32 device tensor of
    num_slots*HV*dk*dv elements) or over a fresh zeroed tensor."""
    import torch
    if storage is None:
        storage = torch.zeros((num_slots, num_v_heads, dk, dv), dtype=torch.float32, device=device)
    if storage.dtype != torch.float32 or not storage.is_contiguous():
        raise ValueError("pool storage must be a contiguous float32 tensor")
    if storage.numel() != num_slots * num_v_heads * dk * dv:
        raise ValueError("pool storage has the wrong number of elements")
    h = c_void_p()
    _check(load_library().gdn_state_pool_create(num_slots, num_v_heads, dk, dv,
                                                c_void_p(storage.data_ptr()), byref(h)))
    return StatePool(h.value, storage, num_slots, num_v_heads, dk, dv)


def gdn_state_pool_alloc(pool: StatePool, n: int):
    out = (c_int32 * max(n, 1))()
    _check(load_library().gdn_state_pool_alloc(c_void_p(pool.handle), n, out))
    return [int(out[i]) for i in range(n)]


def gdn_state_pool_retain(pool: StatePool, slot: int) -> None:
    _check(load_library().gdn_state_pool_retain(c_void_p(pool.handle), slot))


def gdn_state_pool_release(pool: StatePool, slot: int) -> None:
    _check(load_library().gdn_state_pool_release(c_void_p(pool.handle), slot))


def gdn_state_pool_cow(pool: StatePool, src: int) -> int:
    d = c_int32(-1)
    _check(load_library().gdn_state_pool_cow(c_void_p(pool.handle), src, byref(d)))
    return int(d.value)


def gdn_state_pool_validate(pool: StatePool, src, dst) -> None:
    s = np.ascontiguousarray(np.asarray(src, np.int32))
    d = np.ascontiguousarray(np.asarray(dst, np.int32))
    if s.shape != d.shape:
        raise ValueError("src and dst tables differ in length")
    _check(load_library().gdn_state_pool_validate(
        c_void_p(pool.handle), len(s), s.ctypes.data_as(POINTER(c_int32)), d.ctypes.data_as(POINTER(c_int32))))


def gdn_state_pool_refcount(pool: StatePool, slot: int) -> int:
    r = c_int32()
    _check(load_library().gdn_state_pool_refcount(c_void_p(pool.handle), slot, byref(r)))
    return int(r.value)


def gdn_state_pool_num_free(pool: StatePool) -> int:
    r = c_int32()
    _check(load_library().gdn_state_pool_num_free(c_void_p(pool.handle), byref(r)))
    return int(r.value)


def gdn_state_pool_capacity(pool: StatePool) -> int:
    r = c_int32()
    _check(load_library().gdn_state_pool_capacity(c_void_p(pool.handle), byref(r)))
    return int(r.value)


# ---------------------------------------------------------------------------
# launches
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}; q, k, v, o must be float32 or bfloat16")


def _dev(t, name, dtype=None):
    import torch
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_void_p(s.cuda_stream)


def gdn_decode_step(pool: StatePool, q, k, v, g, beta, o, src_slots, dst_slots, *, scale=None,
                    l2_eps: float = 1e-6, err_flag=None, stream=None) -> None:
    """One decode token per request. q, k: [B, HK, dk]; v, o: [B, HV, dv]
    (all float32 or all bfloat16); g, beta: float32 [B, HV]; src/dst: int32
    device [B]. Enqueued on ``stream`` (default: the current stream)."""
    a = decode_args(q, k, v, g, beta, o, src_slots, dst_slots, scale=scale, l2_eps=l2_eps, err_flag=err_flag)
    _check(load_library().gdn_decode_step(c_void_p(pool.handle), byref(a), _stream(stream)))


def decode_args(q, k, v, g, beta, o, src_slots, dst_slots, *, scale=None, l2_eps: float = 1e-6,
                err_flag=None) -> DecodeArgs:
    """The gdn_decode_args struct for these tensors (shapes as in
    gdn_decode_step). The struct holds raw addresses: the tensors must stay
    alive while it, or a graph recorded from it, is in use."""
    import torch
    B, HK, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    dt = _dtype_code(q)
    for t, n in ((k, "k"), (v, "v"), (o, "o")):
        if t.dtype != q.dtype:
            raise ValueError(f"{n} must have q's dtype")
    if tuple(k.shape) != (B, HK, dk) or tuple(v.shape) != (B, HV, dv) or tuple(o.shape) != (B, HV, dv):
        raise ValueError("q/k/v/o shapes disagree")
    if tuple(g.shape) != (B, HV) or tuple(beta.shape) != (B, HV):
        raise ValueError("g and beta must be [B, HV]")
    if src_slots.numel() != B or dst_slots.numel() != B:
        raise ValueError("slot tables must have B entries")
    a = DecodeArgs()
    a.batch, a.num_k_heads, a.num_v_heads, a.dk, a.dv, a.dtype = B, HK, HV, dk, dv, dt
    a.q, a.k, a.v, a.o = _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o")
    a.g, a.beta = _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    a.src_slots, a.dst_slots = _dev(src_slots, "src_slots", torch.int32), _dev(dst_slots, "dst_slots", torch.int32)
    a.scale = float(dk ** -0.5 if scale is None else scale)
    a.l2_eps = float(l2_eps)
    a.err_flag = _dev(err_flag, "err_flag", torch.int32)
    return a


class DecodeGraph:
    """A recorded list of decode launches (gdn_decode_graph_*).

    ``entries``: DecodeArgs structs (see decode_args), replayed in order;
    ``storages``: optional list of float32 device tensors of the pool's shape
    (None entries use the pool's storage). The graph keeps references to
    ``keep`` (the tensors the structs point at) so they outlive it."""

    def __init__(self, pool: StatePool, entries, storages=None, *, layer_events: bool = False, keep=()):
        n = len(entries)
        arr = (DecodeArgs * max(n, 1))(*entries)
        import torch
        st = None
        if storages is not None:
            if len(storages) != n:
                raise ValueError("storages must have one entry per launch")
            want = pool.num_slots * pool.num_v_heads * pool.dk * pool.dv
            for t in storages:
                if t is not None and t.numel() != want:
                    raise ValueError("every storage must hold the pool's num_slots * HV * dk * dv floats")
            st = (c_void_p * n)(*[None if t is None else _dev(t, "storage", torch.float32) for t in storages])
        h = c_void_p()
        flags = GDN_GRAPH_LAYER_EVENTS if layer_events else 0
        _check(load_library().gdn_decode_graph_create(c_void_p(pool.handle), n, arr, st, flags, byref(h)))
        self.handle = h.value
        self.num_entries = n
        self._keep = (pool, list(keep), list(storages or []))

    def launch(self, stream=None) -> None:
        _check(load_library().gdn_decode_graph_launch(c_void_p(self.handle), _stream(stream)))

    def poll(self):
        """(replays finished, err_flag bits of the last one), read from host memory."""
        n, f = ctypes.c_uint32(), c_int32()
        _check(load_library().gdn_decode_graph_poll(c_void_p(self.handle), byref(n), byref(f)))
        return int(n.value), int(f.value)

    def wait_entry(self, entry: int, stream=None) -> None:
        _check(load_library().gdn_decode_graph_wait_entry(c_void_p(self.handle), int(entry), _stream(stream)))

    def sync_entry(self, entry: int) -> None:
        _check(load_library().gdn_decode_graph_sync_entry(c_void_p(self.handle), int(entry)))

    def close(self) -> None:
        if self.handle:
            load_library().gdn_decode_graph_destroy(c_void_p(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PrefixCache:
    """Radix tree over token ids whose nodes own slot checkpoints of `pool`
    (the C library's logical prefix cache). Close it before the pool."""

    def __init__(self, pool: StatePool):
        h = c_void_p()
        _check(load_library().gdn_prefix_cache_create(c_void_p(pool.handle), byref(h)))
        self.handle = h.value
        self.pool = pool

    @staticmethod
    def _tokens(tokens):
        t = np.ascontiguousarray(np.asarray(tokens, np.int32))
        return t, t.ctypes.data_as(POINTER(c_int32))

    def insert(self, tokens, slot: int) -> bool:
        """The cache retains `slot` as the state after `tokens`; False if that
        prefix already had a checkpoint (nothing changes then)."""
        t, ptr = self._tokens(tokens)
        out = c_int32()
        _check(load_library().gdn_prefix_cache_insert(c_void_p(self.handle), ptr, len(t), int(slot), byref(out)))
        return bool(out.value)

    def match(self, tokens):
        """(length, slot) of the longest checkpointed prefix, (0, -1) on a
        miss; a hit retains the slot for the caller."""
        t, ptr = self._tokens(tokens)
        n, s = c_int32(), c_int32()
        _check(load_library().gdn_prefix_cache_match(c_void_p(self.handle), ptr, len(t), byref(n), byref(s)))
        return n.value, s.value

    def evict(self, want_free: int) -> int:
        out = c_int32()
        _check(load_library().gdn_prefix_cache_evict(c_void_p(self.handle), int(want_free), byref(out)))
        return out.value

    def size(self) -> int:
        out = c_int32()
        _check(load_library().gdn_prefix_cache_size(c_void_p(self.handle), byref(out)))
        return out.value

    def close(self) -> None:
        if self.handle:
            load_library().gdn_prefix_cache_destroy(c_void_p(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gdn_state_pool_pack(pool: StatePool, slots, buffer, *, err_flag=None, stream=None) -> None:
    """buffer[i] <- pool tile of slots[i] (zero state for a negative slot).
    slots: int32 device [n]; buffer: float32 device [n, HV, dk, dv]."""
    import torch
    n = slots.numel()
    if tuple(buffer.shape) != (n, pool.num_v_heads, pool.dk, pool.dv):
        raise ValueError("buffer must be [n, HV, dk, dv]")
    _check(load_library().gdn_state_pool_pack(
        c_void_p(pool.handle), n, _dev(slots, "slots", torch.int32), _dev(buffer, "buffer", torch.float32),
        _dev(err_flag, "err_flag", torch.int32), _stream(stream)))


def gdn_state_pool_unpack(pool: StatePool, slots, buffer, *, err_flag=None, stream=None) -> None:
    """pool tile of slots[i] <- buffer[i] (negative slots skipped; the others
    distinct). slots: int32 device [n]; buffer: float32 device [n, HV, dk, dv]."""
    import torch
    n = slots.numel()
    if tuple(buffer.shape) != (n, pool.num_v_heads, pool.dk, pool.dv):
        raise ValueError("buffer must be [n, HV, dk, dv]")
    _check(load_library().gdn_state_pool_unpack(
        c_void_p(pool.handle), n, _dev(slots, "slots", torch.int32), _dev(buffer, "buffer", torch.float32),
        _dev(err_flag, "err_flag", torch.int32), _stream(stream)))


def gdn_decode_verify(pool: StatePool, q, k, v, g, beta, o, src_slots, dst_slots, *, draft_lens=None,
                      scale=None, l2_eps: float = 1e-6, err_flag=None, stream=None) -> None:
    """Speculative-decode verification, K draft tokens per request in one
    launch. q, k: [B, K, HK, dk]; v, o: [B, K, HV, dv] (all float32 or all
    bfloat16); g, beta: float32 [B, K, HV]; src: int32 device [B]; dst: int32
    device [B, K] (state after draft token i -> dst[b, i], < 0 = not stored);
    draft_lens: optional int32 device [B] (tokens verified per request).
    Enqueued on ``stream`` (default: the current stream)."""
    import torch
    B, K, HK, dk = q.shape
    HV, dv = v.shape[2], v.shape[3]
    dt = _dtype_code(q)
    for t, n in ((k, "k"), (v, "v"), (o, "o")):
        if t.dtype != q.dtype:
            raise ValueError(f"{n} must have q's dtype")
    if tuple(k.shape) != (B, K, HK, dk) or tuple(v.shape) != (B, K, HV, dv) or tuple(o.shape) != (B, K, HV, dv):
        raise ValueError("q/k/v/o shapes disagree")
    if tuple(g.shape) != (B, K, HV) or tuple(beta.shape) != (B, K, HV):
        raise ValueError("g and beta must be [B, K, HV]")
    if src_slots.numel() != B or tuple(dst_slots.shape) != (B, K):
        raise ValueError("src must have B entries and dst shape [B, K]")
    if draft_lens is not None and draft_lens.numel() != B:
        raise ValueError("draft_lens must have B entries")
    a = VerifyArgs()
    a.batch, a.num_draft, a.num_k_heads, a.num_v_heads, a.dk, a.dv, a.dtype = B, K, HK, HV, dk, dv, dt
    a.q, a.k, a.v, a.o = _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o")
    a.g, a.beta = _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    a.src_slots, a.dst_slots = _dev(src_slots, "src_slots", torch.int32), _dev(dst_slots, "dst_slots", torch.int32)
    a.draft_lens = _dev(draft_lens, "draft_lens", torch.int32)
    a.scale = float(dk ** -0.5 if scale is None else scale)
    a.l2_eps = float(l2_eps)
    a.err_flag = _dev(err_flag, "err_flag", torch.int32)
    _check(load_library().gdn_decode_verify(c_void_p(pool.handle), byref(a), _stream(stream)))


def _prefill_args(pool, q, k, v, g, beta, o, cu_seqlens, cu_seqlens_host, src_slots, dst_slots,
                  scale, l2_eps, err_flag, ckpt_slots=None, *, full=True):
    """The gdn_prefill_args struct. With ``full`` every tensor is checked
    against the shapes q [T, HK, dk] and v [T, HV, dv] fix (k, o, g, beta, the
    slot tables, the device cu_seqlens): a wrong size would otherwise reach
    the kernels as a raw pointer. ``full=False`` (workspace sizing) reads only
    the shapes of q and v."""
    import torch
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [T, HK, dk] and v [T, HV, dv]")
    T, HK, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    if v.shape[0] != T:
        raise ValueError("q and v must have the same number of tokens")
    host = np.ascontiguousarray(np.asarray(cu_seqlens_host, np.int32))
    if host.ndim != 1 or host.size < 1:
        raise ValueError("cu_seqlens_host must be a 1-D table of N + 1 offsets")
    N = len(host) - 1
    if full:
        _dtype_code(q)
        for t, n in ((k, "k"), (v, "v"), (o, "o")):
            if t.dtype != q.dtype:
                raise ValueError(f"{n} must have q's dtype")
        if tuple(k.shape) != (T, HK, dk):
            raise ValueError(f"k must be [T, HK, dk] = {(T, HK, dk)}")
        if tuple(o.shape) != (T, HV, dv):
            raise ValueError(f"o must be [T, HV, dv] = {(T, HV, dv)}")
        for t, n in ((g, "g"), (beta, "beta")):
            if t is None or tuple(t.shape) != (T, HV):
                raise ValueError(f"{n} must be float32 [T, HV] = {(T, HV)}")
        if src_slots is None or dst_slots is None or src_slots.numel() != N or dst_slots.numel() != N:
            raise ValueError(f"src_slots and dst_slots must have N = {N} entries")
        if cu_seqlens is None or cu_seqlens.numel() != N + 1:
            raise ValueError(f"cu_seqlens (device) must have N + 1 = {N + 1} entries")
        if err_flag is not None and err_flag.numel() < 1:
            raise ValueError("err_flag must hold one int32")
    a = PrefillArgs()
    a.num_seqs, a.total_tokens, a.chunk_size = N, T, 64
    a.num_k_heads, a.num_v_heads, a.dk, a.dv = HK, HV, dk, dv
    a.dtype = _dtype_code(q)
    a.cu_seqlens = _dev(cu_seqlens, "cu_seqlens", torch.int32) if cu_seqlens is not None else None
    a.cu_seqlens_host = host.ctypes.data
    if T > 0 and full:
        a.q, a.k, a.v, a.o = _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o")
        a.g, a.beta = _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    if src_slots is not None:
        a.src_slots = _dev(src_slots, "src_slots", torch.int32)
        a.dst_slots = _dev(dst_slots, "dst_slots", torch.int32)
    a.scale = float(dk ** -0.5 if scale is None else scale)
    a.l2_eps = float(l2_eps)
    a.err_flag = _dev(err_flag, "err_flag", torch.int32)
    if ckpt_slots is not None:
        nchunks = int(np.sum((np.diff(host.astype(np.int64)) + 63) // 64))
        if ckpt_slots.numel() != nchunks:
            raise ValueError(f"ckpt_slots must have {nchunks} entries (one per 64-token chunk)")
        a.ckpt_slots = _dev(ckpt_slots, "ckpt_slots", torch.int32)
    return a, host


def gdn_prefill_workspace_bytes(pool: StatePool, q, v, cu_seqlens_host) -> int:
    """Workspace bytes for a prefill of these shapes (q: [T, HK, dk], v: [T, HV, dv])."""
    a, host = _prefill_args(pool, q, q, v, None, None, v, None, cu_seqlens_host, None, None, None, 1e-6, None,
                            full=False)
    n = c_size_t()
    _check(load_library().gdn_prefill_workspace_bytes(c_void_p(pool.handle), byref(a), byref(n)))
    return int(n.value)


def gdn_prefill_chunked(pool: StatePool, q, k, v, g, beta, o, cu_seqlens, cu_seqlens_host, src_slots,
                        dst_slots, *, workspace=None, scale=None, l2_eps: float = 1e-6, err_flag=None,
                        ckpt_slots=None, stream=None):
    """Varlen chunked prefill. q, k: [T, HK, dk]; v, o: [T, HV, dv], all
    bfloat16 (chunk form on bf16 matrix cores) or all float32 (the same chunk
    form on fp32 matrix cores); g, beta: float32 [T, HV]; cu_seqlens: int32 device [N+1] with its host
    mirror; src/dst: int32 device [N]. ``workspace``: a uint8 device tensor of
    at least gdn_prefill_workspace_bytes (allocated here if None).
    ``ckpt_slots``: optional int32 device [sum ceil(len / 64)], the slot that
    receives the state after each 64-token chunk (-1: none). Returns the
    workspace tensor so callers can reuse it."""
    import torch
    a, host = _prefill_args(pool, q, k, v, g, beta, o, cu_seqlens, cu_seqlens_host, src_slots, dst_slots,
                            scale, l2_eps, err_flag, ckpt_slots)
    n = c_size_t()
    _check(load_library().gdn_prefill_workspace_bytes(c_void_p(pool.handle), byref(a), byref(n)))
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().gdn_prefill_chunked(c_void_p(pool.handle), byref(a), c_void_p(workspace.data_ptr()),
                                              nbytes, _stream(stream)))
    if stream is not None and stream != torch.cuda.current_stream():
        # the caching allocator ties a block to the stream it was made on;
        # the kernels use it on `stream`, so it must not be reused before
        # that stream's work ends
        workspace.record_stream(stream)
    return workspace


def gdn_prefill_chunked_static(pool: StatePool, q, k, v, g, beta, o, cu_seqlens, cu_seqlens_host, src_slots,
                               dst_slots, *, scale=None, l2_eps: float = 1e-6, err_flag=None, ckpt_slots=None,
                               stream=None) -> None:
    """gdn_prefill_chunked on the library's static per-GPU workspace (no
    device allocation anywhere, here or in the library). Same arguments and
    results; calls needing more than GDN_PREFILL_STATIC_WORKSPACE_BYTES of
    workspace raise. Calls whose work overlaps on one GPU share that workspace
    and must be serialised by the caller."""
    a, host = _prefill_args(pool, q, k, v, g, beta, o, cu_seqlens, cu_seqlens_host, src_slots, dst_slots,
                            scale, l2_eps, err_flag, ckpt_slots)
    _check(load_library().gdn_prefill_chunked_static(c_void_p(pool.handle), byref(a), _stream(stream)))
