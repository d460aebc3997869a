"""Seeded synthetic workloads for compressed-KV sparse attention.

This package holds shapes and random draws only.  It contains none of the
method's arithmetic (no projection, pooling, normalisation, rotation,
scoring, selection or attention): every value it produces is either a random
draw or a bit pattern assembled from random draws.  Both the CPU oracle
(``oracle/``) and the HIP path read the same bytes from here.
"""
from .configs import CONFIGS, LayerShape, get_config, flash_ratio  # noqa: F401
from .gen import (  # noqa: F401
    DecodeInputs,
    LayerWeights,
    PrefillInputs,
    make_decode_inputs,
    make_layer_weights,
    make_prefill_inputs,
    row_bytes,
)
