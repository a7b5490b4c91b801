"""Seeded synthetic workloads for the MoE layer forward.

This package only draws random inputs (router logits, activations, weights)
and lays them out in the storage formats the layer consumes.  It holds none of
the layer's own arithmetic: the weight codes are produced with torch's
float8 casts (a library primitive), and routing is the softmax/top-k recipe a
router would hand the layer.  Both the GPU path and the CPU oracle consume the
same arrays.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    LayerInputs,
    MoEShape,
    make_activations,
    make_fp8_block_weights,
    make_layer_inputs,
    make_mxfp8_weights,
    make_routing,
    token_groups_balanced,
)
