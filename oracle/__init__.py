"""CPU oracle for the MLA decode step (mla_oracle), the latent-cache writer
(cache_writer), the DSA sparse decode step (dsa), TPLA decode (tpla), grouped MLA
decode (grouped) and MHA-mode prefill (prefill).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
calls it, and it shares no code with the HIP library.
"""
from .mla_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    build_selectors,
    decode_storage,
    e4m3_code_to_f64,
    gather_sequence,
    gqa_decode,
    mla_decode_absorbed,
    mla_decode_explicit,
    oracle_from_inputs,
    softmax,
)
