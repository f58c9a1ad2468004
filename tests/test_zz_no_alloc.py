"""gdn_prefill_chunked_static (the prefill on the library's static per-GPU
workspace, for callers that cannot allocate device memory) against
gdn_prefill_chunked (caller workspace) on the same inputs, through the C ABI:
outputs and every slot of the pool must match bit for bit, over two calls in
a row on the shared static array, the second with a smaller input (so the
first call's leftovers sit in the array), in bf16 and in fp32. The rejection
of a call whose workspace exceeds the array is checked on the CPU.
"""

import sys

import numpy as np
import pytest

from hybrid_linear_attention_02_amd import gdn
from hybrid_linear_attention_02_amd.workloads import BF16, F32, prefill_workload
from _util import to_dev


def _call(entry, pw, src, dst):
    import torch
    tk = pw.tokens
    dt = pw.dtype
    storage = torch.from_numpy(pw.pool.copy()).cuda()
    pool = gdn.gdn_state_pool_create(pw.num_slots, pw.HV, pw.dk, pw.dv, storage=storage)
    pool.alloc(pw.num_slots)
    v = to_dev(tk.v, dt)
    o = torch.full_like(v, float("nan"))
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
    args = (pool, to_dev(tk.q, dt), to_dev(tk.k, dt), v, to_dev(tk.g, "f32"), to_dev(tk.beta, "f32"), o,
            torch.from_numpy(pw.cu_seqlens).cuda(), pw.cu_seqlens, i32(src), i32(dst))
    if entry == "static":
        gdn.gdn_prefill_chunked_static(*args, scale=pw.dk ** -0.5)
    else:
        gdn.gdn_prefill_chunked(*args, scale=pw.dk ** -0.5)
    torch.cuda.synchronize()
    pool.close()
    return o.cpu(), storage.cpu()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_static_workspace_matches_caller_workspace_two_calls(dtype):
    import torch
    calls = [
        # a 2,500-token sequence (split into segments by the planner for bf16),
        # resuming from a pool state, packed with two shorter ones
        dict(lengths=[2500, 700, 33], src=[0, -1, 1], dst=[3, 4, 5], seed=801),
        # then a smaller call: the array still holds the first call's data
        dict(lengths=[200, 64], src=[2, -1], dst=[3, 4], seed=802),
    ]
    for i, c in enumerate(calls):
        print(f"[no-alloc] {dtype} call {i}: lengths {c['lengths']}", file=sys.stderr, flush=True)
        pw = prefill_workload(f"static_ws_{dtype}_{i}", seed=c["seed"], lengths=c["lengths"], HK=2, HV=4, dk=128,
                              dv=128, dtype=dtype, num_slots=6, pool_sigma=0.05, src=c["src"], g_range=(1e-3, 0.1))
        o_s, st_s = _call("static", pw, c["src"], c["dst"])
        o_w, st_w = _call("workspace", pw, c["src"], c["dst"])
        assert not torch.isnan(o_s.float()).any(), "static-workspace call left outputs unwritten"
        assert torch.equal(o_s.view(torch.int16) if dtype == BF16 else o_s.view(torch.int32),
                           o_w.view(torch.int16) if dtype == BF16 else o_w.view(torch.int32)), \
            f"call {i}: outputs differ from the caller-workspace entry point"
        assert torch.equal(st_s.view(torch.int32), st_w.view(torch.int32)), f"call {i}: pool differs"
        np.testing.assert_array_equal(st_s.numpy()[[j for j in range(6) if j not in c["dst"]]],
                                      pw.pool[[j for j in range(6) if j not in c["dst"]]])


def test_static_workspace_rejects_a_call_beyond_its_size():
    """A 8192-token call at 16/32 heads needs about 87 MiB of workspace, more
    than the 64 MiB array: the call fails before anything reaches the GPU."""
    from ctypes import byref, c_size_t, c_void_p
    lib = gdn.load_library()
    buf = np.zeros(16, np.float32)
    h = c_void_p()
    assert lib.gdn_state_pool_create(2, 32, 128, 128, c_void_p(buf.ctypes.data), byref(h)) == gdn.GDN_OK
    cuh = np.asarray([0, 8192], np.int32)
    a = gdn.PrefillArgs()
    a.num_seqs, a.total_tokens = 1, 8192
    a.cu_seqlens, a.cu_seqlens_host = buf.ctypes.data, cuh.ctypes.data
    a.chunk_size, a.num_k_heads, a.num_v_heads, a.dk, a.dv, a.dtype = 64, 16, 32, 128, 128, gdn.GDN_DTYPE_BF16
    for f in ("q", "k", "v", "g", "beta", "o", "src_slots", "dst_slots"):
        setattr(a, f, buf.ctypes.data)
    a.scale, a.l2_eps = 128 ** -0.5, 1e-6
    n = c_size_t()
    assert lib.gdn_prefill_workspace_bytes(h, byref(a), byref(n)) == gdn.GDN_OK
    assert n.value > gdn.GDN_PREFILL_STATIC_WORKSPACE_BYTES
    assert lib.gdn_prefill_chunked_static(h, byref(a), None) == gdn.GDN_E_INVALID
    assert "static" in gdn.gdn_last_error()
    lib.gdn_state_pool_destroy(h)
