"""CPU oracle for the routed-MoE expert FFN over low-bit experts.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The
library itself (``bit_routed_moe_amd``) never does: it has no CPU fallback.

What it computes is the plain definition of one MoE layer, evaluated in fp64
with numpy, one token (and one expert pair) at a time:

  router  logits = W_r x with the bf16 router matrix (fp64 product)
  route   softmax over the router logits, top-k with lowest-index tie-break,
          renormalised weights over the k selected experts
  permute stable expert-major order of the (token, slot) pairs
  FFN     per pair: h = silu(W_g x) * (W_u x), o = W_d h, with the routed
          weights decoded exactly from their Q2K-style, Q4K-style or MXFP4
          bytes
  shared  the same SwiGLU FFN with bf16 weights, for every token
  combine y = shared + sum_j w_j o_j

The pages fix only which tensors are low-bit: the routed experts alone are
quantized, while the shared expert, the projections and routing stay at
original precision (hysenlabs "DwarfStar実地分析", section
"GGUFの対応範囲は意図的に狭い"; README mirror "DS4 分布式Shell客户端",
section "模型下载").  Everything else (formats' field order, router function,
activation) is the reading written out in each function's docstring.

It shares no code with the HIP path: nothing here imports the library, its
headers or its build, and the library imports nothing from here.  Inputs come
from ``synth`` (seeded generators with no layer arithmetic).
"""
from .formats import (fp16_to_float64, q2k_decode, q2k_decode_matrix, q4k_decode_matrix, e2m1_to_float64,
                      mxfp4_decode_matrix, bf16_bits_to_float64, fp32_round,
                      bf16_bits_from_fp32, e4m3_round, mxfp8_quantize)
from .moe import (router_logits, route, route_softmax_chain, permute, silu, swiglu_ffn, decode_routed,
                  decode_shared, expert_outputs, shared_outputs, combine, forward,
                  forward_expert_outer, dense_mixture)

__all__ = [
    "fp16_to_float64", "q2k_decode", "q2k_decode_matrix", "q4k_decode_matrix", "e2m1_to_float64",
    "mxfp4_decode_matrix", "bf16_bits_to_float64", "fp32_round", "bf16_bits_from_fp32",
    "e4m3_round", "mxfp8_quantize",
    "router_logits", "route", "route_softmax_chain", "permute", "silu", "swiglu_ffn", "decode_routed",
    "decode_shared", "expert_outputs", "shared_outputs", "combine", "forward",
    "forward_expert_outer", "dense_mixture",
]
