"""Seeded synthetic clustered output-embedding workloads.

This package generates inputs only: the embedding table E, the centroids C,
the cluster-to-token table C2T and the query hidden states h.  It holds none
of the retrieval head's arithmetic (no scoring, selection, quantisation or
sampling), so that both the HIP path and the CPU oracle can be fed from it
without sharing any of the method's code.
"""

from .clustered import (  # noqa: F401
    SHAPES,
    Problem,
    Shape,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_graded_queries,
    make_problem,
)
