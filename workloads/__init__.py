"""Seeded synthetic inputs shared by the HIP library's tests/bench and the oracle.

This module only draws random arrays and rounds them to the storage type; it
holds none of the method's arithmetic (no attention, importance, selection or
projection).  Both sides read the arrays it returns; neither side's code lives
here.

Random numbers come from ``numpy.random.Generator(PCG64(seed))`` with the draw
order Q, K, V, positions, cluster parameters.  Arrays meant to be stored in
bfloat16 are drawn in fp32 and rounded to the nearest bfloat16 (ties to even);
the rounded values are the inputs of both sides.

The workloads stand in for the long-context retrieval suites the pages
evaluate on (RULER-v2, MRCR-v2, NoLiMa, GraphWalks), which are not available:
needles model scattered evidence tokens and clusters model retrievable
spans, at the context lengths the pages use (32k pretraining, 256k
post-training, 1M cost analysis).
"""

from .generators import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits,
    bf16_bits_to_f32,
    make_bridge_inputs,
    make_decode_inputs,
    make_prefill_inputs,
)
