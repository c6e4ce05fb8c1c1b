"""Seeded synthetic inputs for the GPTQ layer path.

This package holds only random-number generation and array shaping. It
contains none of the quantizer's arithmetic, so both the HIP path (through
its tests and the benchmark) and the float64 oracle may draw their inputs
from it without sharing any part of the method.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    activation_chunks,
    activations,
    n_outliers,
    outlier_channels,
    token_scales,
    weights,
)
