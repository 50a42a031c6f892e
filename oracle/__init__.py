"""CPU oracle for shared-KV attention (test infrastructure, float64 NumPy).

Imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg; the library itself never imports it and has no CPU path.
"""
from .kv_oracle import (  # noqa: F401
    PAGE, PoolShape, append, append_aliasing, attend, bf16_to_f64, decode, decode_from_logical, decode_private, extend, fetch,
    pack, unpack,
    extend_from_logical, gather, k_offset, pool_elems, tile_elems, tile_start, v_offset,
)
