"""ds4moe_forward_noalloc (forward with its workspace in the library's fixed
per-device array) against ds4moe_forward with a caller workspace: the same
launches, so the outputs must be bit-identical, on consecutive calls whose
second is smaller (the array keeps the first call's contents), across the
three launch sequences (batch 1, GEMV, grouped GEMM), plus a layer checked
against the oracle, and the size limit refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
from synth import LayerSpec, WORKLOADS, make_layer, make_x, make_logits

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, weights, rowwise_rel_err, to_dev, workspace  # noqa: E402


def _both(dl, cfg, T, seed, zipf=None):
    spec = dl.spec
    x = make_x(T, spec.hidden, seed=seed, dtype="bf16").to(DEV)
    logits = make_logits(T, spec.n_experts, seed=seed + 1, zipf_s=zipf).to(DEV)
    y_ref = torch.full((T, spec.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds4.forward(cfg, weights(dl), T, x, logits, y_ref, workspace(cfg, T))
    y = torch.full((T, spec.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds4.forward_noalloc(cfg, weights(dl), T, x, logits, y)
    torch.cuda.synchronize()
    return x, logits, y, y_ref


def test_noalloc_matches_forward_full_size():
    spec = WORKLOADS["decode"]["spec"]
    print("noalloc full size: T=32 (grouped), then T=6 (GEMV), then T=1 (batch 1)", flush=True)
    dl = make_layer(spec, seed=7150, device=DEV)
    cfg = config(spec, algo="auto")
    for T, path in ((32, 2), (6, 0), (1, 1)):
        assert ds4.forward_path(cfg, T) == path
        assert ds4.workspace_bytes(cfg, T) <= ds4.forward_noalloc_max_bytes()
        _, _, y, y_ref = _both(dl, cfg, T, seed=40 + T, zipf=1.1 if T == 32 else None)
        assert torch.isfinite(y.float()).all()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), T


def test_noalloc_small_layer_oracle_and_repeat():
    """A small layer twice in a row (the second call smaller), each against
    forward bit for bit and the oracle to the bf16 bar."""
    spec = LayerSpec(768, 384, 16, 4, 256, "q2k")
    layer = make_layer(spec, seed=7151, device="cpu")
    dl = to_dev(layer)
    cfg = config(spec, algo="auto")
    for T in (300, 37):
        x, logits, y, y_ref = _both(dl, cfg, T, seed=60 + T)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), T
        r = oracle.forward(layer, x.float().cpu().numpy(), logits.cpu().numpy())
        ref = np.stack([r["y"][t] for t in range(T)])
        assert rowwise_rel_err(y.float().cpu().numpy(), ref) <= 2e-2


def test_noalloc_refuses_oversize():
    """A call whose workspace would exceed the fixed array is refused on the
    host (nothing launched: y keeps its contents)."""
    spec = WORKLOADS["prefill"]["spec"]
    cfg = config(spec, algo="auto")
    T = 4096
    assert ds4.workspace_bytes(cfg, T) > ds4.forward_noalloc_max_bytes()
    z = torch.zeros(16, dtype=torch.uint8, device=DEV)
    w = ds4.make_weights(z, z, z, sh_gate=z, sh_up=z, sh_down=z)
    y = torch.full((4,), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ds4.Ds4MoeError) as ei:
        ds4.forward_noalloc(cfg, w, T, z, z, y)
    assert ei.value.status == -5
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
