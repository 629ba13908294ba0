"""CPU oracle for the KV-shared early-exit decoder -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it, and no
product code path falls back to it.
"""
from .river_oracle import (  # noqa: F401
    EXIT_COPY, EXIT_INT4, RiverOracle, Shape, apply_rope, attention, bf16_from_f32,
    bf16_from_f64, cosine_rows, decoder_layer, dequantize_int4, greedy, linear, lm_head,
    quantize_int4, rmsnorm, rope_tables, silu,
)
