"""fp64 CPU oracle for MLA decode, causal prefill (naive and absorbed) and the
cache-row producer.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product path (the HIP library and its binding)
never imports, loads or calls anything in this package.
"""
from .oracle import (  # noqa: F401
    OracleError,
    absorb_q,
    build,
    cache_rows,
    decode_absorbed,
    decode_latent,
    decode_naive,
    fold_value_output,
    kv_cache_bytes,
    max_threads,
    output_proj,
    prefill_absorbed,
    prefill_naive,
    rope,
    set_threads,
)
