"""Seeded synthetic inputs for the GDN state-update workloads.

This module only draws random numbers and lays them out. It holds none of the
state-update arithmetic, so both the HIP path (tests, bench) and the fp64
oracle consume exactly the same arrays from it.

Recipe (the workload shapes follow the agentic multi-turn description on the
TokenSpeed pages -- 24-ai.news (English), section "Agentic workload results":
a 50K-token first turn, then 800-token turns -- and the head shape of a
16 key-head / 32 value-head GDN layer with 128 x 128 state tiles):

* q, k, v ~ N(0, 1), drawn in float32. q and k are L2-normalised in float32
  per (token, key head). bf16 inputs are then rounded to bfloat16 with
  round-to-nearest-even and kept as uint16 bit patterns; both sides consume the
  rounded values.
* g = -U(lo, hi) per (token, value head), float32 (default lo=0.01, hi=0.5).
* beta = sigmoid(N(0, 1)) per (token, value head), float32.
* Pool tiles ~ N(0, sigma) float32.
* Generator: numpy.random.Generator(PCG64(seed)); draw order is pool, slots,
  then q, k, v, g, beta (per decode step, or once per prefill batch).
* Raw (un-normalised) q and k, for the cases that exercise the kernels' own
  L2 normalisation: instead of normalising, every (token, key head) row of q
  and of k is rescaled to a norm drawn log-uniformly in [lo, hi] (one extra
  draw per tensor, after beta), and the rows with (t + j) % 11 == 3 (k) or
  (t + j) % 13 == 5 (q), t the token and j the key head, get norm 1e-4, where
  the normalisation's epsilon dominates.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite draws, so NaN handling is not needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def _normalise_rows_f32(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


@dataclass
class Tokens:
    """One batch of per-token inputs. q, k, v are float32 arrays for F32 and
    uint16 bfloat16 bit patterns for BF16; g and beta are always float32."""
    dtype: str
    q: np.ndarray          # [T, HK, dk]
    k: np.ndarray          # [T, HK, dk]
    v: np.ndarray          # [T, HV, dv]
    g: np.ndarray          # [T, HV]
    beta: np.ndarray       # [T, HV]


TINY_ROW_NORM = 1e-4


def _rescale_rows(rng, x, lo, hi, tiny_mod, tiny_rem):
    """Rows of x [T, HK, d] rescaled to norms log-uniform in [lo, hi]; rows
    with (t + j) % tiny_mod == tiny_rem to norm TINY_ROW_NORM."""
    T, HK, _ = x.shape
    target = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(T, HK))).astype(np.float32)
    tt, jj = np.meshgrid(np.arange(T), np.arange(HK), indexing="ij")
    target[(tt + jj) % tiny_mod == tiny_rem] = np.float32(TINY_ROW_NORM)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n * target[..., None]).astype(np.float32)


def draw_tokens(rng, T, HK, HV, dk, dv, dtype, *, g_range=(0.01, 0.5),
                beta_mode="sigmoid", normalise_qk=True, v_scale=1.0, raw_norms=None) -> Tokens:
    q = rng.standard_normal((T, HK, dk), dtype=np.float32)
    k = rng.standard_normal((T, HK, dk), dtype=np.float32)
    v = (rng.standard_normal((T, HV, dv), dtype=np.float32) * np.float32(v_scale)).astype(np.float32)
    lo, hi = g_range
    g = (-rng.uniform(lo, hi, size=(T, HV))).astype(np.float32)
    if beta_mode == "sigmoid":
        beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, HV))))).astype(np.float32)
    else:
        beta = np.full((T, HV), float(beta_mode), np.float32)
    if raw_norms is not None:
        if normalise_qk:
            raise ValueError("raw_norms needs normalise_qk=False")
        q = _rescale_rows(rng, q, raw_norms[0], raw_norms[1], 13, 5)
        k = _rescale_rows(rng, k, raw_norms[0], raw_norms[1], 11, 3)
    elif normalise_qk:
        q = _normalise_rows_f32(q)
        k = _normalise_rows_f32(k)
    if dtype == BF16:
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif dtype != F32:
        raise ValueError(dtype)
    return Tokens(dtype, q, k, v, g, beta)


@dataclass
class DecodeWorkload:
    name: str
    B: int
    HK: int
    HV: int
    dk: int
    dv: int
    dtype: str
    num_slots: int
    pool: np.ndarray                 # [num_slots, HV, dk, dv] float32
    src: np.ndarray                  # [B] int32 source slots of the first step
    steps: list = field(default_factory=list)   # list[Tokens], T = B each


@dataclass
class PrefillWorkload:
    name: str
    HK: int
    HV: int
    dk: int
    dv: int
    dtype: str
    num_slots: int
    pool: np.ndarray                 # [num_slots, HV, dk, dv] float32
    cu_seqlens: np.ndarray           # [N+1] int32
    src: np.ndarray                  # [N] int32 (-1 = zero initial state)
    tokens: Tokens = None
    chunk: int = 64


@dataclass
class VerifyWorkload:
    """K draft tokens per request for speculative-decode verification; token
    (b, i) is row b * K + i of `tokens`."""
    name: str
    B: int
    K: int
    HK: int
    HV: int
    dk: int
    dv: int
    dtype: str
    num_slots: int
    pool: np.ndarray                 # [num_slots, HV, dk, dv] float32
    src: np.ndarray                  # [B] int32
    tokens: Tokens = None            # T = B * K


def verify_workload(name, *, seed, B, K, HK, HV, dk, dv, dtype, num_slots, pool_sigma,
                    src=None, g_range=(0.01, 0.5), beta_mode="sigmoid", raw_norms=None) -> VerifyWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = (rng.standard_normal((num_slots, HV, dk, dv), dtype=np.float32) * np.float32(pool_sigma)).astype(np.float32)
    if src is None:
        src = rng.permutation(num_slots)[:B]
    src = np.asarray(src, np.int32)
    toks = draw_tokens(rng, B * K, HK, HV, dk, dv, dtype, g_range=g_range, beta_mode=beta_mode,
                       normalise_qk=raw_norms is None, raw_norms=raw_norms)
    return VerifyWorkload(name, B, K, HK, HV, dk, dv, dtype, num_slots, pool, src, toks)


def decode_workload(name, *, seed, B, HK, HV, dk, dv, dtype, num_slots, pool_sigma,
                    steps, src=None, g_range=(0.01, 0.5), beta_mode="sigmoid", raw_norms=None) -> DecodeWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = (rng.standard_normal((num_slots, HV, dk, dv), dtype=np.float32) * np.float32(pool_sigma)).astype(np.float32)
    if src is None:
        src = rng.permutation(num_slots)[:B]
    src = np.asarray(src, np.int32)
    toks = [draw_tokens(rng, B, HK, HV, dk, dv, dtype, g_range=g_range, beta_mode=beta_mode,
                        normalise_qk=raw_norms is None, raw_norms=raw_norms)
            for _ in range(steps)]
    return DecodeWorkload(name, B, HK, HV, dk, dv, dtype, num_slots, pool, src, toks)


def prefill_workload(name, *, seed, lengths, HK, HV, dk, dv, dtype, num_slots, pool_sigma=0.0,
                     src=None, g_range=(0.01, 0.5), beta_mode="sigmoid", v_scale=1.0,
                     raw_norms=None) -> PrefillWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    if pool_sigma > 0:
        pool = (rng.standard_normal((num_slots, HV, dk, dv), dtype=np.float32) * np.float32(pool_sigma)).astype(np.float32)
    else:
        pool = np.zeros((num_slots, HV, dk, dv), np.float32)
    N = len(lengths)
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, np.int64))
    if src is None:
        src = -np.ones(N, np.int32)
    src = np.asarray(src, np.int32)
    toks = draw_tokens(rng, int(cu[-1]), HK, HV, dk, dv, dtype, g_range=g_range,
                       beta_mode=beta_mode, v_scale=v_scale, normalise_qk=raw_norms is None,
                       raw_norms=raw_norms)
    return PrefillWorkload(name, HK, HV, dk, dv, dtype, num_slots, pool, cu, src, toks)


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def tiny_decode(steps=8) -> DecodeWorkload:
    """1 request, 1 key head, 2 value heads, 16 x 16 fp32, 4-slot pool
    ~N(0, 0.1), source slot 1, 8 steps, seed 0."""
    return decode_workload("tiny_decode_fp32_16x16", seed=0, B=1, HK=1, HV=2, dk=16, dv=16,
                           dtype=F32, num_slots=4, pool_sigma=0.1, steps=steps, src=[1])


def batched_decode(steps=100, B=64) -> DecodeWorkload:
    """64 requests, 16/32 heads, 128 x 128 bf16, 256-slot pool ~N(0, 0.05),
    sources a random permutation of the pool, seed 1."""
    return decode_workload("batched_decode_bf16_b64_h32_128x128", seed=1, B=B, HK=16, HV=32,
                           dk=128, dv=128, dtype=BF16, num_slots=256, pool_sigma=0.05,
                           steps=steps)


def chunked_prefill(T=8192) -> PrefillWorkload:
    """One sequence of 8192 bf16 tokens, 16/32 heads, 128 x 128, zero initial
    state, seed 2."""
    return prefill_workload("chunked_prefill_bf16_t8192_h32_128x128", seed=2, lengths=[T], HK=16,
                            HV=32, dk=128, dv=128, dtype=BF16, num_slots=2)


def multiturn_resume(tokens_per_seq=800, decode_steps=32):
    """4 checkpoint slots ~N(0, 0.05), 16 sequences (4 per checkpoint) of 800
    bf16 tokens each, then 32 decode steps at B = 16; seed 3. The checkpoints
    occupy slots 0..3 of a 64-slot pool; sequence n resumes from slot n // 4."""
    rng_seed = 3
    pw = prefill_workload("multiturn_resume_bf16_16x800_h32_128x128", seed=rng_seed,
                          lengths=[tokens_per_seq] * 16, HK=16, HV=32, dk=128, dv=128,
                          dtype=BF16, num_slots=64, pool_sigma=0.05,
                          src=np.repeat(np.arange(4), 4).astype(np.int32))
    rng = np.random.Generator(np.random.PCG64(rng_seed + 1000))
    dec = [draw_tokens(rng, 16, 16, 32, 128, 128, BF16) for _ in range(decode_steps)]
    return pw, dec


def long_packed_lengths(first=50_000, n_short=16, lo=1024, hi=16384, seed=4) -> list:
    """Sequence lengths of the long/packed workload: the first sequence, then
    n_short lengths uniform in [lo, hi] (inclusive)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [first] + [int(x) for x in rng.integers(lo, hi, size=n_short, endpoint=True)]


def long_packed_prefill(first=50_000, n_short=16, lo=1024, hi=16384, seed=4,
                        g_range=(0.01, 0.5)) -> PrefillWorkload:
    """One 50,000-token sequence plus 16 sequences with lengths uniform in
    [1024, 16384] (inclusive), packed via cu_seqlens, zero initial states.
    ``g_range`` other than the default gives a weak-decay variant of the same
    shape (the lengths do not change)."""
    lengths = long_packed_lengths(first, n_short, lo, hi, seed)
    name = "long_packed_prefill_bf16_h32_128x128" + ("" if tuple(g_range) == (0.01, 0.5) else "_weak_decay")
    return prefill_workload(name, seed=seed + 100, lengths=lengths,
                            HK=16, HV=32, dk=128, dv=128, dtype=BF16, num_slots=len(lengths) + 1,
                            g_range=g_range)


def spec_verify(B=64, K=4) -> VerifyWorkload:
    """Speculative-decode verification at the batched-decode head shape: 64
    requests, 4 draft tokens each, 16/32 heads, 128 x 128 bf16, seed 5. The
    pool has room for the sources and one destination per draft position
    (B (K + 1) slots, ~N(0, 0.05)); sources are a random permutation."""
    return verify_workload("spec_verify_bf16_b64_k4_h32_128x128", seed=5, B=B, K=K, HK=16, HV=32, dk=128, dv=128,
                           dtype=BF16, num_slots=B * (K + 1), pool_sigma=0.05)
