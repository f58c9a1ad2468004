"""The Python binding's own argument checks, on the CPU (no GPU call is made:
every case fails in the binding before a pointer reaches the library).

A wrong tensor size would otherwise reach the kernels as a raw pointer, which
the C ABI cannot see; the binding checks each tensor of a prefill call
against the shapes q [T, HK, dk] and v [T, HV, dv] fix.
"""

import numpy as np
import pytest
import torch

from hybrid_linear_attention_02_amd import gdn

T, HK, HV, DK, DV, N = 70, 2, 4, 64, 32, 2
CU = np.array([0, 30, 70], np.int32)


def _args(**change):
    bf = torch.bfloat16
    a = dict(q=torch.zeros(T, HK, DK, dtype=bf), k=torch.zeros(T, HK, DK, dtype=bf),
             v=torch.zeros(T, HV, DV, dtype=bf), g=torch.zeros(T, HV), beta=torch.zeros(T, HV),
             o=torch.zeros(T, HV, DV, dtype=bf), cu_seqlens=torch.from_numpy(CU), cu_seqlens_host=CU,
             src_slots=torch.zeros(N, dtype=torch.int32), dst_slots=torch.ones(N, dtype=torch.int32))
    a.update(change)
    return a


CASES = [
    ("k_dtype", dict(k=torch.zeros(T, HK, DK)), "k must have q's dtype"),
    ("v_dtype", dict(v=torch.zeros(T, HV, DV)), "v must have q's dtype"),
    ("o_dtype", dict(o=torch.zeros(T, HV, DV)), "o must have q's dtype"),
    ("k_short", dict(k=torch.zeros(T - 1, HK, DK, dtype=torch.bfloat16)), "k must be"),
    ("k_heads", dict(k=torch.zeros(T, HK + 1, DK, dtype=torch.bfloat16)), "k must be"),
    ("o_short", dict(o=torch.zeros(T - 5, HV, DV, dtype=torch.bfloat16)), "o must be"),
    ("o_width", dict(o=torch.zeros(T, HV, DV // 2, dtype=torch.bfloat16)), "o must be"),
    ("v_tokens", dict(v=torch.zeros(T - 1, HV, DV, dtype=torch.bfloat16)), "same number of tokens"),
    ("g_shape", dict(g=torch.zeros(T, HV - 1)), "g must be"),
    ("beta_shape", dict(beta=torch.zeros(T + 1, HV)), "beta must be"),
    ("src_short", dict(src_slots=torch.zeros(N - 1, dtype=torch.int32)), "src_slots and dst_slots"),
    ("dst_long", dict(dst_slots=torch.zeros(N + 1, dtype=torch.int32)), "src_slots and dst_slots"),
    ("cu_device_short", dict(cu_seqlens=torch.from_numpy(CU[:-1].copy())), "cu_seqlens"),
    ("cu_device_missing", dict(cu_seqlens=None), "cu_seqlens"),
    ("q_rank", dict(q=torch.zeros(T, HK * DK, dtype=torch.bfloat16)), "q must be"),
]


@pytest.mark.parametrize("cid,change,msg", CASES, ids=[c[0] for c in CASES])
def test_prefill_binding_rejects_mismatched_tensor(cid, change, msg):
    a = _args(**change)
    with pytest.raises(ValueError, match=msg):
        gdn.gdn_prefill_chunked(None, a["q"], a["k"], a["v"], a["g"], a["beta"], a["o"], a["cu_seqlens"],
                                a["cu_seqlens_host"], a["src_slots"], a["dst_slots"])


def test_prefill_binding_consistent_host_tensors_reach_the_device_check():
    """Tensors that agree pass the shape checks and stop only at the first
    device-pointer check (these are host tensors)."""
    a = _args()
    with pytest.raises(ValueError, match="device tensor"):
        gdn.gdn_prefill_chunked(None, a["q"], a["k"], a["v"], a["g"], a["beta"], a["o"], a["cu_seqlens"],
                                a["cu_seqlens_host"], a["src_slots"], a["dst_slots"])


def test_library_shares_torchs_hip_runtime():
    """Loading the library first must not put a second HIP runtime into the
    process: in a fresh interpreter that opens libgdn.so before anything
    else, exactly one libamdhip64 is mapped, and it is torch's."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("from hybrid_linear_attention_02_amd import gdn; gdn.load_library(); "
            "print('\\n'.join(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l})))")
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    libs = out.stdout.split()
    import torch
    assert libs == [os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")], libs
