"""GPU parity of the grouped-GEMM (matrix-core) expert FFN against the fp64 oracle.

Tolerance: per-token infinity-norm relative error <= 2e-2 (bf16 path).
Small layers are checked on every token, at token counts that give ragged
16-token tiles, experts above the 160-token chunk limit (split chunks) and
several shared-expert chunks, and a 65,536-token batch on sampled tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import LayerSpec, WORKLOADS, make_layer, make_x, make_logits

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, weights, rowwise_rel_err, to_dev, workspace  # noqa: E402

TOL = 2e-2


def _forward(dl, cfg, T, x, logits):
    y = torch.full((T, dl.spec.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds4.forward(cfg, weights(dl), T, x.to(DEV), logits.to(DEV), y, workspace(cfg, T))
    torch.cuda.synchronize()
    return y


def _check(layer, dl, T, algo="grouped", seed=0, zipf=None, tokens=None):
    spec = layer.spec
    x = make_x(T, spec.hidden, seed=100 + seed, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=200 + seed, zipf_s=zipf)
    y = _forward(dl, config(spec, algo=algo), T, x, logits)
    assert torch.isfinite(y.float()).all()
    r = oracle.forward(layer, x.float().numpy(), logits.numpy(), tokens=tokens)
    toks = sorted(r["y"])
    ref = np.stack([r["y"][t] for t in toks])
    err = rowwise_rel_err(y.float().cpu().numpy()[toks], ref)
    print(f"  T={T} algo={algo} tokens={len(toks)} err={err:.3e}", flush=True)
    return err


SMALL = [
    # name, spec, T
    ("tiny", LayerSpec(256, 128, 8, 2, 0, "q2k"), 16),
    ("tiny_shared", LayerSpec(256, 128, 8, 2, 128, "q2k"), 16),
    ("mx_tiny", LayerSpec(256, 128, 8, 2, 128, "mxfp4"), 16),
    ("ragged", LayerSpec(768, 384, 16, 4, 256, "q2k"), 37),
    ("mx_ragged", LayerSpec(768, 384, 16, 4, 256, "mxfp4"), 37),
    ("one_expert", LayerSpec(512, 256, 1, 1, 0, "q2k"), 5),
    ("k_eq_E", LayerSpec(256, 256, 4, 4, 128, "q2k"), 3),
    # 32 tokens on 2 experts top-2: every chunk (and the shared expert's) is two
    # full tiles, the most the small-batch layout holds
    ("two_full_tiles", LayerSpec(512, 256, 2, 2, 256, "q2k"), 32),
    ("mx_two_full_tiles", LayerSpec(512, 256, 2, 2, 256, "mxfp4"), 32),
    # experts with 200-300 tokens: split into two chunks; shared expert in 3 chunks
    ("split", LayerSpec(512, 256, 4, 2, 256, "q2k"), 500),
    ("mx_split", LayerSpec(512, 256, 4, 2, 256, "mxfp4"), 500),
    # one shared chunk of 12 full tiles
    ("t192", LayerSpec(256, 128, 8, 2, 128, "q2k"), 192),
    # wide rows: several 256-row blocks per down chunk, 16 up row blocks
    ("wide", LayerSpec(2048, 2048, 8, 2, 2048, "q2k"), 96),
]


@pytest.mark.parametrize("name,spec,T", SMALL, ids=[s[0] for s in SMALL])
def test_grouped_small(name, spec, T):
    print(f"grouped small {name} T={T}", flush=True)
    layer = make_layer(spec, seed=300 + len(name), device="cpu")
    assert _check(layer, to_dev(layer), T) <= TOL


def test_grouped_skewed_tile_counts():
    """Zipf-skewed routing over 24 experts: expert loads from 3 to 588 tokens,
    so chunks of 1..11 token tiles and experts split into 2..4 chunks run in
    one launch."""
    spec = LayerSpec(256, 128, 24, 3, 0, "q2k")
    layer = make_layer(spec, seed=77, device="cpu")
    assert _check(layer, to_dev(layer), 700, seed=3, zipf=1.1) <= TOL


def test_grouped_expert_ffn_stage():
    """expert_out rows and shared_out of the grouped kernels against the oracle,
    with routing from the oracle."""
    spec = LayerSpec(512, 256, 8, 2, 256, "q2k")
    T = 150
    layer = make_layer(spec, seed=41, device="cpu")
    dl = to_dev(layer)
    x = make_x(T, spec.hidden, seed=42, dtype="bf16")
    idx, _ = oracle.route(make_logits(T, 8, seed=43).numpy(), 2)
    perm = oracle.permute(idx, 8)
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    cfg = config(spec, algo="grouped")
    eo = torch.full((T * 2, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    so = torch.full((T, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds4.expert_ffn(cfg, weights(dl), T, x.to(DEV), i32(perm["offsets"]), i32(perm["sorted_pair"]),
                   i32(perm["active"]), eo, so, workspace(cfg, T))
    torch.cuda.synchronize()
    o, _ = oracle.expert_outputs(layer, x.float().numpy(), idx)
    ref_eo = np.stack([o[(int(p) // 2, int(p) % 2)] for p in perm["sorted_pair"]])
    assert rowwise_rel_err(eo.float().cpu().numpy(), ref_eo) <= TOL
    s = oracle.shared_outputs(layer, x.float().numpy())
    assert rowwise_rel_err(so.float().cpu().numpy(), np.stack([s[t] for t in range(T)])) <= TOL


def test_grouped_matches_gemv_small():
    """The two bf16 paths agree with each other to the same bar."""
    spec = LayerSpec(768, 384, 16, 4, 256, "q2k")
    T = 64
    dl = to_dev(make_layer(spec, seed=51, device="cpu"))
    x = make_x(T, spec.hidden, seed=52, dtype="bf16")
    logits = make_logits(T, 16, seed=53)
    yg = _forward(dl, config(spec, algo="grouped"), T, x, logits).float().cpu().numpy()
    yv = _forward(dl, config(spec, algo="gemv"), T, x, logits).float().cpu().numpy()
    assert rowwise_rel_err(yg, yv) <= TOL


def test_grouped_deterministic():
    spec = LayerSpec(512, 256, 4, 2, 256, "q2k")
    T = 300
    dl = to_dev(make_layer(spec, seed=61, device="cpu"))
    x = make_x(T, spec.hidden, seed=62, dtype="bf16")
    logits = make_logits(T, 4, seed=63)
    cfg = config(spec, algo="grouped")
    y1 = _forward(dl, cfg, T, x, logits)
    y2 = _forward(dl, cfg, T, x, logits)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# Full-size layers (prefill, batched decode, 2..16-token batches) are checked
# against the oracle in test_gpu_fullsize.py.


@pytest.mark.parametrize("T,algo", [(8, "gemv"), (9, "grouped"), (33, "grouped")])
def test_auto_token_cut(T, algo):
    """AUTO runs the GEMV kernels up to 8 tokens and the grouped GEMM above
    (the small-batch layout to 32 tokens, the prefill layout from 33): its
    output is bit-identical to the forced choice.  (A dispatch property, not
    parity: the full-size 2..16-token batches are checked against the oracle
    in test_gpu_fullsize.py.)"""
    spec = LayerSpec(512, 256, 16, 4, 256, "q2k")
    layer = make_layer(spec, seed=300 + T, device="cpu")
    dl = to_dev(layer)
    x = make_x(T, spec.hidden, seed=301, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=302)
    ya = _forward(dl, config(spec, algo="auto"), T, x, logits)
    yf = _forward(dl, config(spec, algo=algo), T, x, logits)
    assert torch.equal(ya.view(torch.int16), yf.view(torch.int16))


def test_grouped_large_batch_sampled():
    """65,536 tokens (524,288 pairs) on a 512/256 layer with 64 experts top-8
    and a shared expert: the blocked permutation over 512 token blocks, about
    2,800 chunks in the plan, the persistent work queues; sampled tokens
    (both ends and an expert's run) against the oracle, and the whole output
    finite."""
    spec = LayerSpec(512, 256, 64, 8, 256, "q2k")
    T = 65536
    layer = make_layer(spec, seed=500, device="cpu")
    dl = to_dev(layer)
    print(f"large batch T={T}", flush=True)
    assert _check(layer, dl, T, algo="auto", seed=11, tokens=[0, 1, 777, 32768, 65534, 65535]) <= TOL
