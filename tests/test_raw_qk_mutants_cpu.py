"""The raw-q/k GPU cases must catch a kernel that gets the normalisation
wrong: on the CPU, an oracle with one planted slip in the normalisation
stands in for such a kernel, and the bar of the GPU test (`compare` of
_raw_qk_cases.py) must reject its results against the true oracle on every
case. The slips: no normalisation at all, k or q alone left raw, eps dropped,
and eps added to the norm instead of to the sum of squares.
"""

import inspect

import numpy as np
import pytest

import oracle
import oracle.gdn_oracle as G
from _raw_qk_cases import cases, compare, reference

CASES = cases()

MUTANTS = [
    ("no_normalisation", "gated_delta_token",
     "kh = l2_normalize(k, eps)\n    qt = l2_normalize(q, eps) * scale",
     "kh = np.asarray(k, np.float64)\n    qt = np.asarray(q, np.float64) * scale"),
    ("k_raw", "gated_delta_token", "kh = l2_normalize(k, eps)", "kh = np.asarray(k, np.float64)"),
    ("q_raw", "gated_delta_token", "qt = l2_normalize(q, eps) * scale", "qt = np.asarray(q, np.float64) * scale"),
    ("eps_dropped", "l2_normalize", "keepdims=True) + eps)", "keepdims=True))"),
    ("eps_on_the_norm", "l2_normalize", "np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
     "(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)"),
]


def _mutant(name, old, new):
    src = inspect.getsource(getattr(G, name))
    assert src.count(old) == 1, f"{name}: the text to replace must occur exactly once"
    ns = dict(vars(G))
    exec(compile(src.replace(old, new), f"<mutant of {name}>", "exec"), ns)
    return ns[name]


def _result_of(case, monkeypatch, mutant):
    _, name, old, new = mutant
    with monkeypatch.context() as m:
        fn = _mutant(name, old, new)
        for mod in (G, oracle):
            if hasattr(mod, name):
                m.setattr(mod, name, fn)
        return reference(case)


@pytest.fixture(scope="module")
def refs():
    return {c.id: reference(c) for c in CASES}


@pytest.mark.parametrize("case", CASES, ids=[c.id for c in CASES])
def test_true_oracle_meets_its_own_bar(case, refs):
    compare(case, refs[case.id], refs[case.id])


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
@pytest.mark.parametrize("case", CASES, ids=[c.id for c in CASES])
def test_bar_rejects_planted_normalisation_slip(case, mutant, refs, monkeypatch):
    bad = _result_of(case, monkeypatch, mutant)
    with pytest.raises(AssertionError):
        compare(case, bad, refs[case.id])


@pytest.mark.parametrize("factor", [0.7, 0.9, 1.1])
def test_bf16_bar_rejects_scaled_outputs_at_workload_magnitudes(factor):
    """At the 8192-token workload's input distribution outputs stay below
    about 0.06, where the 2e-2 max-abs bar alone would pass a 0.7x output
    scale. The normwise guard of the shared check must reject 0.7x, 0.9x and
    1.1x, and accept the oracle's own outputs rounded to bf16."""
    from hybrid_linear_attention_02_amd.workloads import chunked_prefill, f32_to_bf16_bits
    from oracle import bf16_bits_to_f64, recurrent_sequence
    from _util import check_outputs
    pw = chunked_prefill(T=256)
    tk = pw.tokens
    o_ref, _ = recurrent_sequence(np.zeros((2, 128, 128)), bf16_bits_to_f64(tk.q[:, :1]),
                                  bf16_bits_to_f64(tk.k[:, :1]), bf16_bits_to_f64(tk.v[:, :2]),
                                  tk.g[:, :2], tk.beta[:, :2], 128 ** -0.5, 1e-6)
    assert np.max(np.abs(o_ref)) < 0.1
    rounded = bf16_bits_to_f64(f32_to_bf16_bits(o_ref.astype(np.float32)))
    check_outputs(rounded, o_ref, "bf16", "bf16-rounded oracle")
    assert np.max(np.abs(factor * o_ref - o_ref)) <= 2e-2 or factor != 0.7   # the absolute bar alone passes 0.7x
    with pytest.raises(AssertionError, match="normwise"):
        check_outputs(factor * o_ref, o_ref, "bf16", f"outputs scaled by {factor}")
