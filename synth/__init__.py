"""Seeded synthetic inputs for the NF4 input-gradient GEMM.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no codebook, no quantisation, no dequantisation, no
GEMM).  Both the CPU oracle's tests and the HIP path's tests and benchmark
take their inputs from here, so the two sides see the same bytes.

Workload shapes follow the configurations the subject page's tests and the
fine-tuning use case imply: token count M, layer out-features N (the
reduction dimension of the input gradient) and layer in-features K (the
output dimension), with NF4 blocks of 64 along K.  The RMSNorm backward's inputs (x, gamma, dy)
are drawn here too; its per-row rms is computed by the consumer.
"""

from synth.inputs import (  # noqa: F401
    CONFIGS,
    FULL_STEP_LAYERS,
    FULL_STEP_PROJECTIONS,
    RMS_NORM_SHAPES,
    SKINNY_SHAPES,
    Shape,
    grad_out_normal,
    random_code_bytes,
    random_scales_uniform,
    rms_norm_inputs,
    weights_normal,
)
