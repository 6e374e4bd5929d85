"""Seeded synthetic inputs for the SVDQuant W4A4 linear layer.

This module only draws random numbers with the shapes and value structure of
the layers the method is applied to (FLUX-like linears with activation outlier
channels and a weight that has a steep leading spectrum). It holds none of the
method's arithmetic: no smoothing, no decomposition, no quantization.  Both the
CPU oracle (via the tests) and the GPU benchmark consume what it returns.
"""
from .gen import (  # noqa: F401
    LayerShape, RawLayer, CONFIGS, config_layers, draw_layer, draw_activations,
    draw_weight, draw_bias, fc2_calibration_input, gelu_tanh_f64,
)
