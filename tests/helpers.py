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


def ws_tensor(ws, cfg, T, region, dtype, shape):
    """A view of one stage result inside forward's workspace (see
    ds4moe_workspace_region)."""
    off, n = ds4.workspace_region(cfg, T, region)
    esz = torch.tensor([], dtype=dtype).element_size()
    assert int(np.prod(shape)) * esz == n, (region, shape, n)
    return ws[off:off + n].view(dtype).view(*shape)


def oracle_pairs(layer, x, idx, tokens, mx8=False, workers=12):
    """oracle.expert_outputs for the given tokens, with the experts they touch
    split into disjoint sets evaluated on threads (numpy releases the GIL in
    its array loops; each pair's arithmetic is unchanged).  Returns (o, h)
    dicts keyed by (t, j)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    idx = np.asarray(idx)
    k = idx.shape[1]
    need = sorted({int(idx[t, j]) for t in tokens for j in range(k)})
    W = max(1, min(workers, len(need)))
    groups = [set(need[i::W]) for i in range(W)]
    o, h = {}, {}
    with ThreadPoolExecutor(W) as ex:
        for oo, hh in ex.map(lambda g: oracle.expert_outputs(layer, x, idx, tokens, mx8=mx8, experts=g), groups):
            o.update(oo)
            h.update(hh)
    return o, h


def oracle_y(layer, x, logits, tokens, mx8=False, workers=12):
    """The oracle's layer output for the given tokens (per-token definition:
    route, the tokens' expert pairs, the shared expert, combine), with the
    expert pairs evaluated by ``oracle_pairs``.  Returns (y [len(tokens)][H]
    float64, dict(idx, w, o, h, s))."""
    import oracle
    x = np.asarray(x, dtype=np.float64)
    idx, w = oracle.route(np.asarray(logits)[list(tokens)], layer.spec.top_k)
    # route is per token: rows of the sampled tokens only, re-indexed
    full_idx = np.zeros((x.shape[0], layer.spec.top_k), dtype=np.int64)
    full_w = np.zeros((x.shape[0], layer.spec.top_k))
    full_idx[list(tokens)] = idx
    full_w[list(tokens)] = w
    o, h = oracle_pairs(layer, x, full_idx, tokens, mx8=mx8, workers=workers)
    s = oracle.shared_outputs(layer, x, tokens)
    ys = []
    for t in tokens:
        ys.append(oracle.combine(full_w[t], np.stack([o[(t, j)] for j in range(layer.spec.top_k)]),
                                 None if s is None else s[t]))
    return np.stack(ys), dict(idx=full_idx, w=full_w, o=o, h=h, s=s)
