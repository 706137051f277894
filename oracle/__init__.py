"""CPU oracle of the DiLoCo outer-step merge.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and
by the benchmark's cpu_baseline leg, never by the product path.
"""
from .core import (  # noqa: F401
    CLIP_SIGMAS, FLT_MIN, N_BUCKETS, NoQuorum, broadcast, clip_range, clip_values, codebook,
    dequantize, encode, fragment_plan, histogram, merge, merge_weights, nesterov, normalize_weights,
    outer_cycle, outer_step, pseudo_gradient, quantize_tensor, rda_merge, ring_chunks, ring_message,
    ring_outer_step, ring_sent_chunk, tensor_stats,
)
