"""CPU oracle for KV-cached grouped-query attention (test infrastructure only).

Nothing in the product path may import this package: only the tests, the smoke
check and the CPU-baseline leg of the benchmark call it. See kvc_oracle.py.
"""
from .kvc_oracle import (  # noqa: F401
    DTYPES,
    OracleCache,
    OracleError,
    OracleLatentCache,
    OracleCapacityError,
    bf16_bits_to_f32,
    causal_mask,
    f16_bits_to_f32,
    storage_bytes,
    round_bf16_bits,
    round_f16_bits,
    round_to_storage,
    rope_freqs,
    rope_rotate,
    rope_rotate64,
    storage_bits,
)
