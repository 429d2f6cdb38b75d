"""CPU oracle for LongNet dilated attention (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.
"""
from .dilated import (backward, backward_dq_rows, brute_force_forward, check_patterns, combine, forward,
                      forward_rows, multiplicity, pair_count, row_map, segment_attention,
                      segment_rows, segments)
from .fp8 import dequantize_per_head, e4m3_decode_table, e4m3_encode, quantize_per_head
from .layer import layer_backward, layer_forward, layer_forward_rows

__all__ = ["backward", "backward_dq_rows", "brute_force_forward", "check_patterns", "combine", "forward",
           "forward_rows", "multiplicity", "pair_count", "row_map", "segment_attention",
           "segment_rows", "segments", "layer_backward", "layer_forward",
           "layer_forward_rows", "dequantize_per_head", "e4m3_decode_table", "e4m3_encode",
           "quantize_per_head"]
