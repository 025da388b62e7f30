"""Float64 CPU oracle for the causal softmax attention hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  It shares no
code with the HIP library and the HIP library never calls it.

Every function is pinned by CPU tests against something other than itself
(torch float64 library attention and autograd, finite differences, closed
forms, invariants, brute force, torch's own fp8 decoding).
"""
from .prefill import (gate_prefix, visible_mask, forward, backward, row_stats,
                      forward_rows)
from .decode import (fp8_e4m3fn_to_f64, gather_request_kv, gather_request_gates,
                     decode_paged, prefill_paged, decode_partials, splitk_reduce)
from .cache import e4m3fn_encode, quantize_token_heads, cache_write_fp8

__all__ = ["gate_prefix", "visible_mask", "forward", "backward", "row_stats",
           "forward_rows", "fp8_e4m3fn_to_f64", "gather_request_kv", "gather_request_gates",
           "decode_paged", "prefill_paged", "decode_partials", "splitk_reduce",
           "e4m3fn_encode", "quantize_token_heads", "cache_write_fp8"]
