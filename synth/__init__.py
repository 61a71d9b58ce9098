"""Seeded synthetic layers for the int8 mixed-precision linear.

This package only draws random inputs (fp16 activations with planted outlier
columns, fp16 weights, optional fp16 bias, fp16 upstream gradients) with numpy's PCG64 generator.  It
holds none of the method's arithmetic: no thresholds are applied to decide
anything, nothing is quantized, nothing is multiplied.  Both the CPU oracle's
tests and the GPU path's tests and benchmark draw their inputs from here.
"""

from .layers import (  # noqa: F401
    LayerSpec,
    WORKLOADS,
    layer_specs,
    make_layer,
    make_inputs,
    draw_activations,
    draw_weight,
    draw_bias,
    draw_grad,
)
