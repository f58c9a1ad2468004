"""GPU parity for value-head groups other than two per key head: G = 1
(one value head per key head) and G = 4, through the C ABI, against the fp64
oracle: decode, speculative verify, bf16 and fp32 prefill. The head map is h -> h // G; with two key heads and G = 4 a map
h -> h % HK would read the wrong key head for every value head but the first
of each group."""

import numpy as np
import pytest

from hybrid_linear_attention_02_amd.workloads import BF16, F32, decode_workload, prefill_workload, verify_workload
import test_decode_gpu as D
import test_prefill_gpu as PB
import test_prefill_f32_gpu as PF
import test_verify_gpu as V

pytestmark = pytest.mark.gpu

GROUPS = [(4, 4), (2, 8)]          # (key heads, value heads): G = 1 and G = 4


@pytest.mark.parametrize("hk,hv", GROUPS, ids=["G1", "G4"])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_decode_head_groups(hk, hv, dtype):
    """Six requests, three steps (fresh destination, then in place), 128 x 64
    tiles, every request followed by the oracle."""
    wl = decode_workload(f"groups_{hk}_{hv}", seed=300 + hv + (dtype == BF16), B=6, HK=hk, HV=hv, dk=128,
                         dv=64, dtype=dtype, num_slots=16, pool_sigma=0.05, steps=3)
    D._run(wl, 3)


@pytest.mark.parametrize("hk,hv", GROUPS, ids=["G1", "G4"])
def test_prefill_bf16_head_groups(hk, hv):
    """Ragged, one-token and empty sequences beside a 2,900-token one that the
    planner splits (few heads leave the chip idle), one entry in place; 128 x
    128, bf16."""
    lengths = [300, 64, 0, 1, 2900]
    src = [-1, 0, 1, -1, 2]
    dst = [3, 4, 5, 6, 2]
    pw = prefill_workload(f"groups_{hk}_{hv}", seed=310 + hv, lengths=lengths, HK=hk, HV=hv, dk=128, dv=128,
                          dtype=BF16, num_slots=7, pool_sigma=0.05, src=src, g_range=(1e-3, 5e-2))
    o, st, _ = PB._gpu_prefill(pw, src, dst)
    PB._check(pw, o, st, src, dst)
    np.testing.assert_array_equal(st.cpu().numpy()[:2], pw.pool[:2])


@pytest.mark.parametrize("hk,hv", GROUPS, ids=["G1", "G4"])
def test_prefill_f32_head_groups(hk, hv):
    """fp32 inputs (the chunk form on fp32 matrix cores), 64 x 32 tiles."""
    lengths = [150, 1, 70]
    src = [-1, 0, 1]
    dst = [2, 3, 1]
    pw = prefill_workload(f"f32_groups_{hk}_{hv}", seed=320 + hv, lengths=lengths, HK=hk, HV=hv, dk=64, dv=32,
                          dtype=F32, num_slots=4, pool_sigma=0.05, src=src)
    og, got = PF._run(pw, src, dst)
    PF._check(pw, src, dst, og, got)
    np.testing.assert_array_equal(got[0], pw.pool[0])


@pytest.mark.parametrize("hk,hv", GROUPS, ids=["G1", "G4"])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_verify_head_groups(hk, hv, dtype):
    """Speculative verify of 3 drafts for 4 requests (one partial, one in
    place over its source), 64 x 32 tiles, every stored state checked."""
    B, K = 4, 3
    wl = verify_workload(f"verify_groups_{hk}_{hv}", seed=330 + hv + (dtype == BF16), B=B, K=K, HK=hk, HV=hv,
                         dk=64, dv=32, dtype=dtype, num_slots=B * (K + 1) + 2, pool_sigma=0.3,
                         src=[0, 1, -1, 3], g_range=(1e-3, 0.2))
    dst = (B + 2 + np.arange(B * K)).reshape(B, K).astype(np.int32)
    dst[3, 0] = 3                          # in place over its own source
    lens = np.array([K, 2, K, K], np.int32)
    res, o_ref, new_ref, states = V._run_verify(wl, wl.src, dst, lens)
    assert res["err"] == 0
    n = V._check(wl, res, o_ref, states, dst, np.arange(B), f"verify {dtype} {hk}/{hv}")
    assert n == len(states) > 0
