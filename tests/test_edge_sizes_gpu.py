"""GPU parity at edge sizes, through the C ABI against the fp64 oracle:
thousands of tiny packed sequences in one prefill call (bf16 and fp32 chunk
forms), and a 4096-request decode launch.

Bar as elsewhere (tests/_util.py): fp32 1e-5 normwise, bf16 2e-2 max-abs on
outputs and 1e-2 relative Frobenius on states; skipped sequences and rows
leave their outputs untouched; slots that are not destinations keep their
bytes.
"""

import numpy as np
import pytest

from oracle import decode_step as oracle_decode, prefill as oracle_prefill
from hybrid_linear_attention_02_amd import gdn
from hybrid_linear_attention_02_amd.workloads import BF16, F32, decode_workload, prefill_workload
from _util import as_f64, check_outputs, check_state, out_f64, to_dev

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _torch():
    import torch
    return torch


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_prefill_thousands_of_tiny_sequences(dtype):
    """3000 sequences of 0-3, 63-65 or 130 tokens packed into one call, from
    pool states or zero, with skipped entries and checkpoints: exercises the
    chunk-offset scans, the chunk-to-sequence search and grids of many
    workgroups."""
    torch = _torch()
    rng = np.random.default_rng(71)
    N = 3000
    choices = np.array([0, 1, 2, 3, 63, 64, 65, 130])
    lengths = rng.choice(choices, size=N, p=[0.1, 0.3, 0.2, 0.2, 0.05, 0.05, 0.05, 0.05])
    nchunks = int(np.sum((lengths + 63) // 64))
    NS = 8 + N + nchunks
    src = np.where(rng.random(N) < 0.5, rng.integers(0, 8, size=N), -1).astype(np.int32)
    dst = (8 + np.arange(N)).astype(np.int32)
    dst[rng.random(N) < 0.05] = -1
    # checkpoints after a fifth of the chunks, each to its own slot (the
    # chunk offsets then come from the multi-round scan)
    ckpt = np.where(rng.random(nchunks) < 0.2, 8 + N + np.arange(nchunks), -1).astype(np.int32)
    pw = prefill_workload(f"tiny_many_{dtype}", seed=72, lengths=lengths.tolist(), HK=1, HV=2, dk=32, dv=32,
                          dtype=dtype, num_slots=NS, pool_sigma=0.1, src=src)
    tk = pw.tokens
    storage = torch.from_numpy(pw.pool.copy()).cuda()
    pool = gdn.gdn_state_pool_create(NS, 2, 32, 32, storage=storage)
    pool.alloc(NS)
    pool.validate(src.tolist(), dst.tolist())
    q, k, v = to_dev(tk.q, dtype), to_dev(tk.k, dtype), to_dev(tk.v, dtype)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    o = torch.full(v.shape, float("nan"), dtype=tdt, device="cuda")
    cu = torch.from_numpy(pw.cu_seqlens).cuda()
    gdn.gdn_prefill_chunked(pool, q, k, v, to_dev(tk.g, "f32"), to_dev(tk.beta, "f32"), o, cu, pw.cu_seqlens,
                            torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), scale=32 ** -0.5,
                            l2_eps=EPS, ckpt_slots=torch.from_numpy(ckpt).cuda())
    torch.cuda.synchronize()
    states = {}
    o_ref, _, fin = oracle_prefill(pw.pool, pw.cu_seqlens, src, dst, as_f64(tk.q, dtype), as_f64(tk.k, dtype),
                                   as_f64(tk.v, dtype), tk.g, tk.beta, 32 ** -0.5, EPS, ckpt=ckpt,
                                   ckpt_states=states)
    og = out_f64(o)
    got = storage.cpu().numpy()
    cuh = pw.cu_seqlens
    live = np.zeros(len(og), bool)
    for n in range(N):
        if dst[n] >= 0:
            live[cuh[n]:cuh[n + 1]] = True
    assert np.all(np.isnan(og[~live])), "skipped sequences must stay unwritten"
    check_outputs(og[live], o_ref[live], dtype, "all written tokens")
    for n in range(N):
        if dst[n] >= 0:
            check_state(got[dst[n]], fin[n], dtype, f"seq {n} slot {dst[n]}")
    assert len(states) > 100
    for c, h in states.items():
        check_state(got[ckpt[c]], h, dtype, f"checkpoint {c} slot {ckpt[c]}")
    written = set(dst[dst >= 0].tolist()) | {int(ckpt[c]) for c in states}
    untouched = np.array(sorted(set(range(NS)) - written))
    np.testing.assert_array_equal(got[untouched], pw.pool[untouched])
    pool.close()


def test_decode_4096_requests():
    """One launch over 4096 requests (tiny 16 x 16 fp32 heads), every request
    against the oracle, with padding rows and shared sources."""
    torch = _torch()
    B, NS = 4096, 4096 + 64
    rng = np.random.default_rng(73)
    src = rng.integers(-1, 64, size=B).astype(np.int32)
    dst = (64 + np.arange(B)).astype(np.int32)
    dst[rng.random(B) < 0.03] = -1
    wl = decode_workload("decode_4096", seed=74, B=B, HK=1, HV=2, dk=16, dv=16, dtype=F32, num_slots=NS,
                         pool_sigma=0.2, steps=1, src=src)
    tk = wl.steps[0]
    storage = torch.from_numpy(wl.pool.copy()).cuda()
    pool = gdn.gdn_state_pool_create(NS, 2, 16, 16, storage=storage)
    pool.alloc(NS)
    pool.validate(src.tolist(), dst.tolist())
    o = torch.full((B, 2, 16), float("nan"), device="cuda")
    gdn.gdn_decode_step(pool, to_dev(tk.q, F32), to_dev(tk.k, F32), to_dev(tk.v, F32), to_dev(tk.g, "f32"),
                        to_dev(tk.beta, "f32"), o, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(),
                        scale=0.25, l2_eps=EPS)
    torch.cuda.synchronize()
    o_ref, _, fin = oracle_decode(wl.pool, src, dst, tk.q, tk.k, tk.v, tk.g, tk.beta, 0.25, EPS)
    og = out_f64(o)
    live = dst >= 0
    assert np.all(np.isnan(og[~live]))
    check_outputs(og[live], o_ref[live], F32, "4096 requests")
    got = storage.cpu().numpy()
    for n in np.flatnonzero(live):
        check_state(got[dst[n]], fin[n], F32, f"request {n}")
    np.testing.assert_array_equal(got[:64], wl.pool[:64])
    pool.close()
