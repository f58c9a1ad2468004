"""Host-side tests of libgdn.so: exports, slot bookkeeping, argument checks.

No GPU is needed: the pool's bookkeeping never touches device memory, and every
argument check here fails (or returns early) before anything is enqueued. Fake
"device" addresses are plain aligned host addresses that are never read.
"""

import ctypes
import os
import re
from ctypes import POINTER, byref, c_int32, c_size_t, c_void_p

import numpy as np
import pytest
from hypothesis import settings, strategies as st
from hypothesis.stateful import RuleBasedStateMachine, invariant, precondition, rule

from oracle import SlotPoolModel
from hybrid_linear_attention_02_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build() first")
    return gdn.load_library()


def _fake_storage(nbytes=1 << 12):
    buf = np.zeros(nbytes // 4 + 64, np.float32)
    addr = buf.ctypes.data
    off = (-addr) % 256
    return buf, addr + off


def _make_pool(lib, num_slots=8, hv=2, dk=16, dv=16):
    buf, addr = _fake_storage()
    h = c_void_p()
    assert lib.gdn_state_pool_create(num_slots, hv, dk, dv, c_void_p(addr), byref(h)) == gdn.GDN_OK
    return buf, h


def test_every_declared_symbol_is_exported(lib):
    header = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = set(re.findall(r"^(?:int|const char\*)\s+(gdn_\w+)\s*\(", header, re.M))
    assert declared == set(gdn.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_create_rejects_bad_arguments(lib):
    buf, addr = _fake_storage()
    h = c_void_p()
    cases = [(0, 2, 16, 16, addr), (4, 0, 16, 16, addr), (4, 2, 24, 16, addr), (4, 2, 16, 256, addr),
             (4, 2, 16, 16, None), (4, 2, 16, 16, addr + 4)]
    for ns, hv, dk, dv, p in cases:
        assert lib.gdn_state_pool_create(ns, hv, dk, dv, c_void_p(p), byref(h)) == gdn.GDN_E_INVALID
        assert lib.gdn_last_error() != b""
    assert lib.gdn_state_pool_create(4, 2, 16, 16, c_void_p(addr), None) == gdn.GDN_E_INVALID


def _alloc(lib, h, n):
    out = (c_int32 * max(n, 1))()
    st_ = lib.gdn_state_pool_alloc(h, n, out)
    return st_, ([int(out[i]) for i in range(n)] if st_ == 0 else [])


class PoolMachine(RuleBasedStateMachine):
    """Drive the C++ pool and the Python model with the same operations and
    require identical status codes, slot ids, refcounts and free counts."""

    CAP = 9

    def __init__(self):
        super().__init__()
        self.lib = gdn.load_library()
        self.buf, self.h = _make_pool(self.lib, num_slots=self.CAP)
        self.model = SlotPoolModel(self.CAP)

    def teardown(self):
        self.lib.gdn_state_pool_destroy(self.h)

    slot = st.integers(min_value=-2, max_value=CAP + 1)

    @rule(n=st.integers(min_value=-1, max_value=CAP + 1))
    def alloc(self, n):
        got = _alloc(self.lib, self.h, n)
        assert got == self.model.alloc(n)

    @rule(s=slot)
    def retain(self, s):
        assert self.lib.gdn_state_pool_retain(self.h, s) == self.model.retain(s)

    @rule(s=slot)
    def release(self, s):
        assert self.lib.gdn_state_pool_release(self.h, s) == self.model.release(s)

    @rule(s=slot)
    def cow(self, s):
        d = c_int32(-1)
        st_ = self.lib.gdn_state_pool_cow(self.h, s, byref(d))
        mst, md = self.model.cow(s)
        assert st_ == mst
        if st_ == 0:
            assert d.value == md

    @rule(src=st.lists(slot, min_size=0, max_size=5), data=st.data())
    def validate(self, src, data):
        dst = data.draw(st.lists(self.slot, min_size=len(src), max_size=len(src)))
        s = np.asarray(src, np.int32)
        d = np.asarray(dst, np.int32)
        got = self.lib.gdn_state_pool_validate(self.h, len(s), s.ctypes.data_as(POINTER(c_int32)),
                                               d.ctypes.data_as(POINTER(c_int32)))
        assert got == self.model.validate(src, dst)

    @invariant()
    def counts_agree(self):
        r = c_int32()
        assert self.lib.gdn_state_pool_num_free(self.h, byref(r)) == 0
        assert r.value == self.model.num_free()
        assert self.lib.gdn_state_pool_capacity(self.h, byref(r)) == 0 and r.value == self.CAP
        for s in range(self.CAP):
            assert self.lib.gdn_state_pool_refcount(self.h, s, byref(r)) == 0
            assert r.value == self.model.ref[s]


PoolMachine.TestCase.settings = settings(max_examples=150, stateful_step_count=40, deadline=None)
TestPoolMachine = PoolMachine.TestCase


def test_pool_refcount_query_errors(lib):
    buf, h = _make_pool(lib)
    r = c_int32()
    assert lib.gdn_state_pool_refcount(h, 8, byref(r)) == gdn.GDN_E_INVALID
    assert lib.gdn_state_pool_refcount(h, -1, byref(r)) == gdn.GDN_E_INVALID
    assert lib.gdn_state_pool_num_free(None, byref(r)) == gdn.GDN_E_INVALID
    assert lib.gdn_state_pool_alloc(h, 1, None) == gdn.GDN_E_INVALID
    assert lib.gdn_state_pool_destroy(None) == gdn.GDN_OK
    lib.gdn_state_pool_destroy(h)


# ---------------------------------------------------------------------------
# argument checks of the launching calls (nothing is ever enqueued here)
# ---------------------------------------------------------------------------

def _decode_args(addr, **kw):
    a = gdn.DecodeArgs()
    a.batch, a.num_k_heads, a.num_v_heads, a.dk, a.dv, a.dtype = 4, 1, 2, 16, 16, gdn.GDN_DTYPE_F32
    for f in ("q", "k", "v", "g", "beta", "o", "src_slots", "dst_slots"):
        setattr(a, f, addr)
    a.scale, a.l2_eps, a.err_flag = 0.25, 1e-6, None
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("change,code", [
    (dict(batch=-1), gdn.GDN_E_INVALID),
    (dict(num_k_heads=0), gdn.GDN_E_INVALID),
    (dict(num_k_heads=3, num_v_heads=2), gdn.GDN_E_INVALID),
    (dict(num_v_heads=4, num_k_heads=1), gdn.GDN_E_INVALID),   # pool has HV = 2
    (dict(dk=32), gdn.GDN_E_INVALID),                          # pool has dk = 16
    (dict(dtype=7), gdn.GDN_E_UNSUPPORTED),
    (dict(q=None), gdn.GDN_E_INVALID),
    (dict(dst_slots=None), gdn.GDN_E_INVALID),
    (dict(l2_eps=-1.0), gdn.GDN_E_INVALID),
    (dict(scale=float("inf")), gdn.GDN_E_INVALID),
    ("misaligned_v", gdn.GDN_E_INVALID),
    ("misaligned_g", gdn.GDN_E_INVALID),
])
def test_decode_argument_errors(lib, change, code):
    buf, h = _make_pool(lib)
    _, addr = _fake_storage()
    if change == "misaligned_v":
        a = _decode_args(addr, v=addr + 8)
    elif change == "misaligned_g":
        a = _decode_args(addr, g=addr + 2)
    else:
        a = _decode_args(addr, **change)
    assert lib.gdn_decode_step(h, byref(a), None) == code
    assert len(lib.gdn_last_error()) > 0
    lib.gdn_state_pool_destroy(h)


def test_decode_empty_batch_is_a_no_op(lib):
    buf, h = _make_pool(lib)
    a = _decode_args(None, batch=0)
    assert lib.gdn_decode_step(h, byref(a), None) == gdn.GDN_OK
    assert lib.gdn_decode_step(None, byref(a), None) == gdn.GDN_E_INVALID
    lib.gdn_state_pool_destroy(h)


@pytest.mark.parametrize("case", ["null_pool", "zero_entries", "too_many", "bad_flags", "batch0", "no_err",
                                  "other_err", "bad_entry", "misaligned_storage"])
def test_decode_graph_create_argument_errors(lib, case):
    # every case fails in the host checks, before the library touches HIP
    buf, h = _make_pool(lib)
    _, addr = _fake_storage()
    _, err = _fake_storage()
    n, flags, pool, storages = 2, 0, h, None
    ents = [_decode_args(addr, err_flag=err), _decode_args(addr, err_flag=err)]
    if case == "null_pool":
        pool = None
    elif case == "zero_entries":
        n = 0
    elif case == "too_many":
        n = gdn.GDN_GRAPH_MAX_ENTRIES + 1
    elif case == "bad_flags":
        flags = 2
    elif case == "batch0":
        ents[1].batch = 0
    elif case == "no_err":
        ents[0].err_flag = None
        ents[1].err_flag = None
    elif case == "other_err":
        ents[1].err_flag = err + 4
    elif case == "bad_entry":
        ents[1].dk = 32
    elif case == "misaligned_storage":
        storages = (c_void_p * 2)(None, addr + 4)
    arr = (gdn.DecodeArgs * 2)(*ents)
    out = c_void_p(1234)
    assert lib.gdn_decode_graph_create(pool, n, arr, storages, flags, byref(out)) != gdn.GDN_OK
    assert out.value == 1234
    assert len(lib.gdn_last_error()) > 0
    lib.gdn_state_pool_destroy(h)


def test_decode_graph_null_handles(lib):
    n, f = ctypes.c_uint32(), c_int32()
    assert lib.gdn_decode_graph_poll(None, byref(n), byref(f)) == gdn.GDN_E_INVALID
    assert lib.gdn_decode_graph_launch(None, None) == gdn.GDN_E_INVALID
    assert lib.gdn_decode_graph_wait_entry(None, 0, None) == gdn.GDN_E_INVALID
    assert lib.gdn_decode_graph_sync_entry(None, 0) == gdn.GDN_E_INVALID
    assert lib.gdn_decode_graph_destroy(None) == gdn.GDN_OK


def _verify_args(addr, **kw):
    a = gdn.VerifyArgs()
    a.batch, a.num_draft, a.num_k_heads, a.num_v_heads, a.dk, a.dv = 4, 3, 1, 2, 16, 16
    a.dtype = gdn.GDN_DTYPE_BF16
    for f in ("q", "k", "v", "g", "beta", "o", "src_slots", "dst_slots"):
        setattr(a, f, addr)
    a.draft_lens, a.scale, a.l2_eps, a.err_flag = None, 0.25, 1e-6, None
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("change,code", [
    (dict(batch=-1), gdn.GDN_E_INVALID),
    (dict(num_draft=0), gdn.GDN_E_INVALID),
    (dict(num_draft=65), gdn.GDN_E_INVALID),
    (dict(num_k_heads=3, num_v_heads=2), gdn.GDN_E_INVALID),
    (dict(dv=32), gdn.GDN_E_INVALID),                          # pool has dv = 16
    (dict(dtype=5), gdn.GDN_E_UNSUPPORTED),
    (dict(o=None), gdn.GDN_E_INVALID),
    (dict(src_slots=None), gdn.GDN_E_INVALID),
    (dict(l2_eps=float("nan")), gdn.GDN_E_INVALID),
    ("misaligned_q", gdn.GDN_E_INVALID),
    ("misaligned_lens", gdn.GDN_E_INVALID),
])
def test_verify_argument_errors(lib, change, code):
    buf, h = _make_pool(lib)
    _, addr = _fake_storage()
    if change == "misaligned_q":
        a = _verify_args(addr, q=addr + 4)
    elif change == "misaligned_lens":
        a = _verify_args(addr, draft_lens=addr + 2)
    else:
        a = _verify_args(addr, **change)
    assert lib.gdn_decode_verify(h, byref(a), None) == code
    assert len(lib.gdn_last_error()) > 0
    lib.gdn_state_pool_destroy(h)


def test_verify_empty_batch_is_a_no_op(lib):
    buf, h = _make_pool(lib)
    a = _verify_args(None, batch=0)
    assert lib.gdn_decode_verify(h, byref(a), None) == gdn.GDN_OK
    assert lib.gdn_decode_verify(None, byref(a), None) == gdn.GDN_E_INVALID
    lib.gdn_state_pool_destroy(h)


def test_pack_unpack_argument_errors(lib):
    buf, h = _make_pool(lib)
    _, addr = _fake_storage()
    for fn in (lib.gdn_state_pool_pack, lib.gdn_state_pool_unpack):
        assert fn(h, 0, None, None, None, None) == gdn.GDN_OK                 # nothing to do
        assert fn(None, 1, c_void_p(addr), c_void_p(addr), None, None) == gdn.GDN_E_INVALID
        assert fn(h, -1, c_void_p(addr), c_void_p(addr), None, None) == gdn.GDN_E_INVALID
        assert fn(h, 2, None, c_void_p(addr), None, None) == gdn.GDN_E_INVALID
        assert fn(h, 2, c_void_p(addr), None, None, None) == gdn.GDN_E_INVALID
        assert fn(h, 2, c_void_p(addr), c_void_p(addr + 8), None, None) == gdn.GDN_E_INVALID   # buffer alignment
        assert fn(h, 2, c_void_p(addr + 2), c_void_p(addr), None, None) == gdn.GDN_E_INVALID   # slot table alignment
        assert len(lib.gdn_last_error()) > 0
    lib.gdn_state_pool_destroy(h)


def _prefill_args(addr, cu_host, **kw):
    a = gdn.PrefillArgs()
    a.num_seqs = len(cu_host) - 1
    a.total_tokens = int(cu_host[-1])
    a.cu_seqlens, a.cu_seqlens_host = addr, cu_host.ctypes.data
    a.chunk_size, a.num_k_heads, a.num_v_heads, a.dk, a.dv, a.dtype = 64, 1, 2, 128, 128, gdn.GDN_DTYPE_BF16
    for f in ("q", "k", "v", "g", "beta", "o", "src_slots", "dst_slots"):
        setattr(a, f, addr)
    a.scale, a.l2_eps, a.err_flag = 0.1, 1e-6, None
    for key, val in kw.items():
        setattr(a, key, val)
    return a


def test_prefill_workspace_size_grows_with_chunks(lib):
    buf, h = _make_pool(lib, hv=2, dk=128, dv=128)
    _, addr = _fake_storage()
    sizes = []
    for cu in ([0, 64], [0, 65], [0, 64, 64, 200]):
        cuh = np.asarray(cu, np.int32)
        a = _prefill_args(addr, cuh)
        n = c_size_t()
        assert lib.gdn_prefill_workspace_bytes(h, byref(a), byref(n)) == gdn.GDN_OK
        assert n.value % 256 == 0
        sizes.append(n.value)
    assert sizes[0] < sizes[1] < sizes[2]
    lib.gdn_state_pool_destroy(h)


@pytest.mark.parametrize("change,code", [
    (dict(chunk_size=32), gdn.GDN_E_UNSUPPORTED),
    (dict(dtype=7), gdn.GDN_E_UNSUPPORTED),
    (dict(total_tokens=5), gdn.GDN_E_INVALID),
    (dict(cu_seqlens_host=None), gdn.GDN_E_INVALID),
    (dict(q=None), gdn.GDN_E_INVALID),
    (dict(src_slots=None), gdn.GDN_E_INVALID),
    ("bad_cu", gdn.GDN_E_INVALID),
    ("small_ws", gdn.GDN_E_INVALID),
    ("misaligned_ws", gdn.GDN_E_INVALID),
])
def test_prefill_argument_errors(lib, change, code):
    buf, h = _make_pool(lib, hv=2, dk=128, dv=128)
    _, addr = _fake_storage()
    cuh = np.asarray([0, 10, 70], np.int32)
    ws, ws_addr = _fake_storage(1 << 16)
    ws_bytes = 1 << 15
    if change == "bad_cu":
        bad = np.asarray([0, 80, 70], np.int32)
        a = _prefill_args(addr, bad, total_tokens=70)
    elif change == "small_ws":
        a = _prefill_args(addr, cuh)
        ws_bytes = 256
    elif change == "misaligned_ws":
        a = _prefill_args(addr, cuh)
        ws_addr += 16
    else:
        a = _prefill_args(addr, cuh, **change)
    assert lib.gdn_prefill_chunked(h, byref(a), c_void_p(ws_addr), ws_bytes, None) == code
    assert len(lib.gdn_last_error()) > 0
    lib.gdn_state_pool_destroy(h)


def test_prefill_no_sequences_is_a_no_op(lib):
    buf, h = _make_pool(lib, hv=2, dk=128, dv=128)
    cuh = np.asarray([0], np.int32)
    a = _prefill_args(None, cuh)
    assert lib.gdn_prefill_chunked(h, byref(a), None, 0, None) == gdn.GDN_OK
    lib.gdn_state_pool_destroy(h)


def test_prefill_f32_workspace_holds_offsets_fp32_blocks_and_scale_rows(lib):
    # fp32 inputs run the chunked form on the fp32 MFMA for every pool head
    # shape, never split: the workspace holds the [N+1] chunk and segment
    # offsets, then per (chunk, value head) T and P as ten fp32 16 x 16
    # blocks each and five 64-float scale rows, sections in 256-byte blocks;
    # it does not depend on dk or dv
    up = lambda x: (x + 255) // 256 * 256
    for dk, dv in ((16, 16), (128, 128), (32, 64)):
        buf, h = _make_pool(lib, hv=2, dk=dk, dv=dv)
        _, addr = _fake_storage()
        cuh = np.asarray([0, 64, 64, 200], np.int32)      # 1 + 0 + 3 chunks
        a = _prefill_args(addr, cuh, dk=dk, dv=dv, dtype=gdn.GDN_DTYPE_F32)
        n = c_size_t()
        assert lib.gdn_prefill_workspace_bytes(h, byref(a), byref(n)) == gdn.GDN_OK
        chunks, hv = 4, 2
        assert n.value == 2 * up(4 * 4) + up(4 * chunks * hv * 2 * 10 * 256) + up(4 * chunks * hv * 5 * 64)
        lib.gdn_state_pool_destroy(h)
    # a long fp32 sequence is not split: no segment sections
    buf, h = _make_pool(lib, hv=2, dk=128, dv=128)
    _, addr = _fake_storage()
    cuh = np.asarray([0, 64 * 500], np.int32)
    a = _prefill_args(addr, cuh, dk=128, dv=128, dtype=gdn.GDN_DTYPE_F32)
    n = c_size_t()
    assert lib.gdn_prefill_workspace_bytes(h, byref(a), byref(n)) == gdn.GDN_OK
    assert n.value == 2 * 256 + 4 * 500 * 2 * (2 * 10 * 256 + 5 * 64)
    lib.gdn_state_pool_destroy(h)


def test_prefill_dk16_runs_on_padded_dk32_tiles(lib):
    """bf16 prefill at dk = 16 runs in the dk = 32 kernels (the MFMA k-step):
    its workspace equals a dk = 32 call's, split sections included; other
    chunk sizes stay unsupported."""
    _, addr = _fake_storage()
    cuh = np.asarray([0, 3000, 3090], np.int32)
    sizes = []
    for dk in (16, 32):
        buf, h = _make_pool(lib, hv=2, dk=dk, dv=16)
        a = _prefill_args(addr, cuh, dk=dk, dv=16)
        n = c_size_t()
        assert lib.gdn_prefill_workspace_bytes(h, byref(a), byref(n)) == gdn.GDN_OK
        sizes.append(n.value)
        a = _prefill_args(addr, cuh, dk=dk, dv=16, chunk_size=32)
        assert lib.gdn_prefill_workspace_bytes(h, byref(a), byref(n)) == gdn.GDN_E_UNSUPPORTED
        lib.gdn_state_pool_destroy(h)
    assert sizes[0] == sizes[1]


def _planned_segments(lib, cu, hv, dk, dv):
    """Segments the planner gives a call, read from the workspace size: the
    split sections (end state E and initial state fp32 dk x dv, transition M
    as bf16 high and low dk x dk, per segment and value head) come after the
    offset tables, the T/P fragments and the scale rows; with no split they
    are empty (0 is returned)."""
    buf, h = _make_pool(lib, hv=hv, dk=dk, dv=dv)
    _, addr = _fake_storage()
    cuh = np.asarray(cu, np.int32)
    a = _prefill_args(addr, cuh, num_k_heads=hv // 2, num_v_heads=hv, dk=dk, dv=dv)
    n = c_size_t()
    assert lib.gdn_prefill_workspace_bytes(h, byref(a), byref(n)) == gdn.GDN_OK
    lib.gdn_state_pool_destroy(h)
    up = lambda x: (x + 255) // 256 * 256
    N = len(cu) - 1
    chunks = int(np.sum((np.diff(np.asarray(cu, np.int64)) + 63) // 64))
    base = 2 * up(4 * (N + 1)) + up(2 * chunks * hv * 2 * 64 * 64) + up(4 * chunks * hv * 5 * 64)
    kdk = max(dk, 32)                    # dk = 16 runs on dk = 32 tiles
    per_seg = hv * (8 * kdk * dv + 4 * kdk * kdk)
    extra = n.value - base
    assert extra >= 0 and extra % per_seg == 0
    return extra // per_seg


def test_planner_split_decisions(lib):
    # one 8192-token sequence at 32 value heads: three segments of 43 chunks
    assert _planned_segments(lib, [0, 8192], 32, 128, 128) == 3
    # 16 sequences of 800 tokens fill the chip without a split
    assert _planned_segments(lib, list(range(0, 16 * 800 + 1, 800)), 32, 128, 128) == 0
    # the long/packed workload: the 50,000-token sequence in three segments, the
    # 16 others (at most 256 chunks) whole: 19 segments
    from hybrid_linear_attention_02_amd.workloads import long_packed_lengths
    cu = [0] + [int(x) for x in np.cumsum(long_packed_lengths())]
    assert _planned_segments(lib, cu, 32, 128, 128) == 19
    # few heads leave the chip idle: a 3,000-token sequence is split, also at 64 value columns
    for dk, dv in ((128, 128), (64, 64), (128, 64)):
        assert _planned_segments(lib, [0, 3000, 3090], 4, dk, dv) > 2
    # small heads split too: the state pass's column groups are at most dk wide
    for dk, dv in ((32, 128), (128, 32), (32, 32), (32, 16), (64, 16)):
        assert _planned_segments(lib, [0, 3000, 3090], 4, dk, dv) > 2, (dk, dv)
