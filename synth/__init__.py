"""Seeded synthetic inputs for the routed-MoE expert layer.

This package makes the inputs that both the HIP path and the CPU oracle consume:
activations, router logits (optionally with a Zipf popularity bias), and layer
weights drawn from N(0, 0.02) and *encoded* into the routed-expert formats
(Q2K-style super-blocks, OCP MXFP4) plus bf16 shared-expert weights.

It holds none of the layer's arithmetic: no decoding of the formats, no routing,
no permutation, no FFN, no combine.  The encoders here are the fixture side of
the formats (weights -> bytes); decoding lives separately in ``oracle/`` (CPU)
and in the HIP kernels (GPU), which share no code with each other or with this
package.  Only byte layouts are common, and those are fixed by the format
definitions written out in each decoder.
"""
from .quant import (q2k_encode, mxfp4_encode, q4k_encode, q2k_bytes_per_matrix, mxfp4_bytes_per_matrix,
                    q4k_bytes_per_matrix)
from .layers import (LayerSpec, Layer, make_layer, make_x, make_logits, make_router_w, zipf_bias,
                     WORKLOADS, workload, derive_seed)

__all__ = [
    "q2k_encode", "mxfp4_encode", "q4k_encode", "q2k_bytes_per_matrix", "mxfp4_bytes_per_matrix",
    "q4k_bytes_per_matrix",
    "LayerSpec", "Layer", "make_layer", "make_x", "make_logits", "make_router_w", "zipf_bias",
    "WORKLOADS", "workload", "derive_seed",
]
