"""Helpers shared by the GPU tests: device layers, the ABI structs, the
oracle comparison metric."""
import numpy as np
import torch

import bit_routed_moe_amd as ds4

DEV = torch.device("cuda:0")


def to_dev(layer):
    """A copy of a host layer's tensors on the GPU (same object type)."""
    if layer.device.type == "cuda":
        return layer
    from synth.layers import Layer
    kw = {}
    for f in ("gate", "up", "down", "gate_scales", "up_scales", "down_scales", "sh_gate", "sh_up", "sh_down"):
        t = getattr(layer, f)
        kw[f] = None if t is None else t.to(DEV)
    return Layer(spec=layer.spec, **kw)


def config(spec, act="bf16", algo="auto", mma="bf16"):
    return ds4.make_config(spec.hidden, spec.ffn, spec.n_experts, spec.top_k, spec.shared_ffn,
                           spec.wfmt, act=act, mma=mma, algo=algo)


def weights(dl):
    return ds4.make_weights(dl.gate, dl.up, dl.down, dl.gate_scales, dl.up_scales, dl.down_scales,
                            dl.sh_gate, dl.sh_up, dl.sh_down)


def rowwise_rel_err(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(np.max(np.abs(got - ref), axis=-1) / den))


def workspace(cfg, T):
    return torch.empty(ds4.workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
