"""Cases with raw (un-normalised) q and k, shared by the GPU parity test of
the kernels' own L2 normalisation (test_raw_qk_gpu.py) and its CPU check
against planted mistakes (test_raw_qk_mutants_cpu.py).

The normalisation is part of the rule every kernel applies (k^ = k /
sqrt(|k|^2 + eps), q~ = q / sqrt(|q|^2 + eps) * scale). The GPU parity
workloads elsewhere feed q and k that are already unit-norm, on which a kernel
that skipped the normalisation would still pass. Here every row has a norm
drawn log-uniformly in [0.05, 20], some rows have norm 1e-4 (where eps
decides the result), and eps is 1e-6 or 1e-2.

Each case has a reference runner (`reference`), which runs the fp64 oracle on
the exact inputs the GPU receives, and a comparison (`compare`), which applies
the parity bar to a result: a dict with
  "o":      outputs, NaN where the path leaves them unwritten;
  "states": {slot: [HV, dk, dv]} for every written destination.
The GPU test passes its own results to `compare`; the CPU test passes the
results of an oracle with the normalisation planted wrong and requires
`compare` to fail. No state-update arithmetic lives here.
"""

from dataclasses import dataclass, field

import numpy as np

from oracle import decode_step as oracle_decode, prefill as oracle_prefill, verify_step as oracle_verify
from hybrid_linear_attention_02_amd.workloads import (
    BF16, F32, decode_workload, prefill_workload, verify_workload)
from _util import as_f64, check_outputs, check_state

RAW_NORMS = (0.05, 20.0)


@dataclass
class Case:
    id: str
    kind: str                 # "decode" | "verify" | "prefill"
    dtype: str
    eps: float
    wl: object
    src: list
    dst: list                 # decode/prefill: [N]; verify: [B][K]
    steps: int = 1            # decode only
    lens: list = None         # verify only
    extra: dict = field(default_factory=dict)


def _decode(dtype, eps, dk, dv, seed):
    wl = decode_workload(f"raw_decode_{dtype}_{dk}x{dv}", seed=seed, B=6, HK=2, HV=4, dk=dk, dv=dv, dtype=dtype,
                         num_slots=14, pool_sigma=0.05, steps=6, g_range=(1e-3, 0.05), raw_norms=RAW_NORMS)
    # request 1 starts from the zero state, request 4 shares request 3's source
    src = [0, -1, 2, 3, 3, 5]
    dst = [6, 7, 8, 9, 10, 11]
    return Case(f"decode-{dtype}-{dk}x{dv}-eps{eps:g}", "decode", dtype, eps, wl, src, dst, steps=6)


def _verify(dtype, eps, seed):
    K = 5
    wl = verify_workload(f"raw_verify_{dtype}", seed=seed, B=4, K=K, HK=2, HV=4, dk=128, dv=64, dtype=dtype,
                         num_slots=4 + 4 * K, pool_sigma=0.05, src=[0, 1, 2, 3], g_range=(1e-3, 0.05),
                         raw_norms=RAW_NORMS)
    dst = [[4 + b * K + i for i in range(K)] for b in range(4)]
    dst[2][1] = -1                                   # one draft state not kept
    return Case(f"verify-{dtype}-eps{eps:g}", "verify", dtype, eps, wl, [0, 1, 2, 3], dst, lens=[5, 3, 5, 1])


def _prefill(dtype, eps, lengths, HK, HV, dk, dv, seed, tag):
    n = len(lengths)
    src = [0] + [-1] * (n - 1)
    dst = list(range(1, n + 1))
    wl = prefill_workload(f"raw_prefill_{tag}", seed=seed, lengths=lengths, HK=HK, HV=HV, dk=dk, dv=dv,
                          dtype=dtype, num_slots=n + 1, pool_sigma=0.05, src=src, g_range=(1e-3, 0.05),
                          raw_norms=RAW_NORMS)
    return Case(f"prefill-{tag}-eps{eps:g}", "prefill", dtype, eps, wl, src, dst)


def cases():
    out = []
    for eps in (1e-6, 1e-2):
        e = int(eps < 1e-3)
        out.append(_decode(F32, eps, 64, 32, 700 + e))
        out.append(_decode(F32, eps, 128, 128, 702 + e))
        out.append(_decode(BF16, eps, 128, 128, 704 + e))
        out.append(_decode(BF16, eps, 32, 64, 706 + e))
        out.append(_verify(F32, eps, 710 + e))
        out.append(_verify(BF16, eps, 712 + e))
        out.append(_prefill(F32, eps, [150, 70, 1], 2, 4, 64, 64, 720 + e, "f32"))
        out.append(_prefill(BF16, eps, [200, 70, 1], 2, 4, 128, 128, 722 + e, "bf16"))
        # a 3000-token sequence the planner splits into segments, with a
        # short one packed after it
        out.append(_prefill(BF16, eps, [3000, 100], 1, 2, 128, 128, 724 + e, "bf16_split"))
    return out


# ---------------------------------------------------------------------------

def _decode_tokens(case, step):
    tk = case.wl.steps[step]
    return (as_f64(tk.q, case.dtype), as_f64(tk.k, case.dtype), as_f64(tk.v, case.dtype), tk.g, tk.beta)


def reference(case):
    """The fp64 oracle on the case's exact inputs (bf16 upcast exactly)."""
    wl, dt, scale = case.wl, case.dtype, case.wl.dk ** -0.5
    if case.kind == "decode":
        pool = wl.pool.copy()
        outs = []
        fin = {}
        for step in range(case.steps):
            src = case.src if step == 0 else case.dst
            q, k, v, g, beta = _decode_tokens(case, step)
            o, pool, f = oracle_decode(pool, src, case.dst, q, k, v, g, beta, scale, case.eps)
            outs.append(o)
            fin = {case.dst[n]: h for n, h in f.items()}
        return {"o": np.stack(outs), "states": fin}
    if case.kind == "verify":
        B, K = wl.B, wl.K
        tk = wl.tokens
        shp = lambda x: x.reshape((B, K) + x.shape[1:])
        o, _, st = oracle_verify(wl.pool, case.src, np.asarray(case.dst), case.lens, shp(as_f64(tk.q, dt)),
                                 shp(as_f64(tk.k, dt)), shp(as_f64(tk.v, dt)), shp(tk.g), shp(tk.beta), scale,
                                 case.eps)
        return {"o": o, "states": {case.dst[b][i]: h for (b, i), h in st.items()}}
    tk = wl.tokens
    o, _, fin = oracle_prefill(wl.pool, wl.cu_seqlens, case.src, case.dst, as_f64(tk.q, dt), as_f64(tk.k, dt),
                               as_f64(tk.v, dt), tk.g, tk.beta, scale, case.eps)
    return {"o": o, "states": {case.dst[n]: h for n, h in fin.items()}}


def compare(case, got, ref):
    """The parity bar on one result; raises AssertionError when it is not met.
    Returns the worst output and state errors."""
    dt = case.dtype
    o, o_ref = np.asarray(got["o"], np.float64), np.asarray(ref["o"], np.float64)
    written = ~np.isnan(o_ref)
    assert np.array_equal(~np.isnan(o), written), f"{case.id}: outputs written where the oracle writes none"
    worst_o = 0.0
    if case.kind == "decode":
        for s in range(o_ref.shape[0]):
            worst_o = max(worst_o, check_outputs(o[s], o_ref[s], dt, f"{case.id} step {s}"))
    elif case.kind == "verify":
        for b in range(o_ref.shape[0]):
            m = written[b, :, 0, 0]
            if m.any():
                worst_o = max(worst_o, check_outputs(o[b, m], o_ref[b, m], dt, f"{case.id} request {b}"))
    else:
        cu = case.wl.cu_seqlens
        for n in range(len(case.src)):
            a, b = cu[n], cu[n + 1]
            if b > a:
                worst_o = max(worst_o, check_outputs(o[a:b], o_ref[a:b], dt, f"{case.id} seq {n}"))
    worst_h = 0.0
    assert set(got["states"]) == set(ref["states"]), f"{case.id}: a different set of slots was written"
    for slot, h_ref in ref["states"].items():
        worst_h = max(worst_h, check_state(got["states"][slot], h_ref, dt, f"{case.id} slot {slot}"))
    return worst_o, worst_h
