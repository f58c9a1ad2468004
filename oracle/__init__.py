"""Plain fp64 CPU oracle for the GDN recurrent-state update.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (the HIP library under ``hybrid_linear_attention_02_amd/csrc`` and
its Python binding) never imports, calls or links it, and the two share no code.
"""

from .gdn_oracle import (  # noqa: F401
    GDN_OK,
    GDN_E_INVALID,
    GDN_E_NO_SLOTS,
    GDN_E_SLOT_STATE,
    GDN_E_ALIAS,
    bf16_bits_to_f64,
    l2_normalize,
    gated_delta_token,
    recurrent_sequence,
    chunked_sequence,
    prefill,
    decode_step,
    verify_step,
    state_pack,
    state_unpack,
    SlotPoolModel,
    PrefixCacheModel,
)
