"""End-to-end prefix caching on the GPU: a prefill stores periodic checkpoints,
the logical cache records them, a second request sharing a prefix matches the
deepest one and resumes copy-on-write from it. Its outputs and final state must
equal the oracle running the second request from scratch, and the checkpoints
must stay byte-identical."""

import numpy as np
import pytest

from oracle import prefill as oracle_prefill
from hybrid_linear_attention_02_amd import gdn
from hybrid_linear_attention_02_amd.workloads import BF16, prefill_workload
from _util import as_f64, check_outputs, check_state, out_f64, to_dev

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _prefill(pool, rows, src, dst, ckpt=None):
    """GPU prefill of one sequence given its per-token input rows."""
    import torch
    q, k, v, g, beta = rows
    T = q.shape[0]
    o = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    cu_h = np.array([0, T], np.int32)
    gdn.gdn_prefill_chunked(pool, to_dev(q, BF16), to_dev(k, BF16), to_dev(v, BF16), to_dev(g, "f32"),
                            to_dev(beta, "f32"), o, torch.from_numpy(cu_h).cuda(), cu_h,
                            torch.tensor([src], dtype=torch.int32, device="cuda"),
                            torch.tensor([dst], dtype=torch.int32, device="cuda"), l2_eps=EPS,
                            ckpt_slots=None if ckpt is None else torch.tensor(ckpt, dtype=torch.int32, device="cuda"))
    return o


def test_resume_from_matched_checkpoint():
    import torch
    TA, shared, tail = 320, 256, 100
    # inputs of request A (320 tokens) and of B's own 100 tokens
    w = prefill_workload("prefix_flow", seed=91, lengths=[TA + tail], HK=2, HV=4, dk=128, dv=128, dtype=BF16,
                         num_slots=12, g_range=(1e-3, 0.05))
    t = w.tokens
    rowsA = tuple(x[:TA] for x in (t.q, t.k, t.v, t.g, t.beta))
    rowsB = tuple(np.concatenate([x[:shared], x[TA:]]) for x in (t.q, t.k, t.v, t.g, t.beta))
    rng = np.random.default_rng(5)
    idsA = rng.integers(0, 50000, TA).astype(np.int32)
    idsB = np.concatenate([idsA[:shared], rng.integers(0, 50000, tail).astype(np.int32)])

    storage = torch.zeros((w.num_slots, w.HV, w.dk, w.dv), dtype=torch.float32, device="cuda")
    pool = gdn.gdn_state_pool_create(w.num_slots, w.HV, w.dk, w.dv, storage=storage)
    cache = gdn.PrefixCache(pool)
    dstA, c1, c3 = pool.alloc(3)
    ckpt = [-1] * 5
    ckpt[1], ckpt[3] = c1, c3                                  # states after tokens 128 and 256
    _prefill(pool, rowsA, -1, dstA, ckpt)
    torch.cuda.synchronize()
    assert cache.insert(idsA[:128], c1) and cache.insert(idsA[:shared], c3) and cache.insert(idsA, dstA)
    for s in (dstA, c1, c3):
        pool.release(s)                                        # the cache is now their only holder
    saved = storage.clone()

    n, src = cache.match(idsB)
    assert (n, src) == (shared, c3)
    dstB = pool.cow(src)                                       # shared checkpoint: a fresh slot
    assert dstB not in (dstA, c1, c3)
    oB = _prefill(pool, tuple(x[n:] for x in rowsB), src, dstB)
    torch.cuda.synchronize()
    pool.release(src)                                          # done reading the checkpoint

    o_ref, _, fin = oracle_prefill(np.zeros((w.num_slots, w.HV, w.dk, w.dv), np.float32), [0, shared + tail],
                                   [-1], [0], as_f64(rowsB[0], BF16), as_f64(rowsB[1], BF16),
                                   as_f64(rowsB[2], BF16), rowsB[3], rowsB[4], w.dk ** -0.5, EPS)
    check_outputs(out_f64(oB), o_ref[shared:], BF16, "request B after the shared prefix")
    check_state(storage[dstB].cpu().numpy(), fin[0], BF16, "request B final state")
    for s in (dstA, c1, c3):
        assert torch.equal(storage[s], saved[s]), f"checkpoint slot {s} changed"
    assert cache.size() == 3
    cache.close()
    pool.close()
