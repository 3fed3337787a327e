"""ds4moe_router_logits against the fp64 oracle, through the C ABI.

bf16 x bf16 products are exact in fp32, so the kernels differ from the exact
sum only by fp32 additions; each element must lie within 1e-5 * sum_h
|W_r[e][h] x[t][h]| of the oracle (the worst-case bound for H = 7168 fp32
additions is 4.3e-4 of that sum; random data sits orders of magnitude below
either).  Shapes cover the GEMV kernel (fp32 mode, and up to 16 tokens), the
matrix-core kernel (more tokens: whole and ragged 64 x 64 tiles, expert
counts off the 16-row tile), the degenerate single expert, the largest
expert count, 70,001 tokens, and the 4096-token x 7168 x 256 router on
sampled tokens.
"""
import numpy as np
import pytest
import torch

from synth import LayerSpec, make_router_w, make_x

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
import oracle  # noqa: E402
from helpers import DEV  # noqa: E402

TOL = 1e-5

CASES = [
    # T, H, E, act
    (1, 7168, 256, "bf16"),      # batch-1 decode router
    (5, 256, 8, "bf16"),
    (16, 512, 24, "bf16"),       # the GEMV kernel's largest batch
    (17, 512, 24, "bf16"),       # the matrix-core kernel's smallest
    (64, 256, 64, "bf16"),       # one whole tile
    (300, 1024, 100, "bf16"),    # several tiles, ragged tokens and experts
    (3, 256, 1, "bf16"),         # a single expert
    (3, 512, 1024, "bf16"),      # the largest expert count
    (40, 768, 33, "f32"),        # fp32 mode, three token blocks
    (1, 7168, 256, "f32"),
]


def _cfg(H, E, act):
    return ds4.make_config(H, 128, E, 1, 0, "q2k", act=act)


def _run(T, H, E, act, seed):
    x = make_x(T, H, seed=seed, dtype=act)
    w = make_router_w(E, H, seed=seed + 1)
    out = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    ds4.router_logits(_cfg(H, E, act), T, x.to(DEV), w.to(DEV), out)
    torch.cuda.synchronize()
    return x.double().numpy(), w.double().numpy(), out


def _check(got, x, w):
    ref = oracle.router_logits(x, w)
    mag = np.abs(x) @ np.abs(w).T
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= TOL * mag), float(np.max(err / mag))


@pytest.mark.parametrize("T,H,E,act", CASES, ids=[f"T{c[0]}_H{c[1]}_E{c[2]}_{c[3]}" for c in CASES])
def test_router_logits_match_oracle(T, H, E, act):
    print(f"router T={T} H={H} E={E} {act}", flush=True)
    x, w, out = _run(T, H, E, act, seed=500 + T)
    _check(out.cpu().numpy(), x, w)


def test_router_logits_deterministic():
    T, H, E = 200, 1024, 96
    x = make_x(T, H, seed=520).to(DEV)
    w = make_router_w(E, H, seed=521).to(DEV)
    cfg = _cfg(H, E, "bf16")
    a = torch.empty((T, E), dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    ds4.router_logits(cfg, T, x, w, a)
    ds4.router_logits(cfg, T, x, w, b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_router_logits_full_size_sampled():
    """4096 tokens, 7168 x 256: the launch the router workload times; the
    oracle checks 96 sampled tokens (every expert)."""
    T, H, E = 4096, 7168, 256
    print(f"router full T={T}", flush=True)
    x, w, out = _run(T, H, E, "bf16", seed=530)
    rows = np.random.default_rng(531).choice(T, size=96, replace=False)
    rows = np.concatenate([rows, [0, 63, 64, T - 1]])
    _check(out.cpu().numpy()[rows], x[rows], w)


def test_router_then_route_matches_oracle_route():
    """The projection feeds ds4moe_route: routing the kernel's logits picks
    the experts the oracle's route picks from those same logits."""
    spec = LayerSpec(7168, 2048, 256, 8, 0, "q2k")
    T = 33
    x = make_x(T, spec.hidden, seed=540).to(DEV)
    w = make_router_w(spec.n_experts, spec.hidden, seed=541).to(DEV)
    cfg = ds4.make_config(spec.hidden, spec.ffn, spec.n_experts, spec.top_k, 0, "q2k")
    logits = torch.empty((T, spec.n_experts), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, spec.top_k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, spec.top_k), dtype=torch.float32, device=DEV)
    ds4.router_logits(cfg, T, x, w, logits)
    ds4.route(cfg, T, logits, idx, tw)
    torch.cuda.synchronize()
    ref_idx, _ = oracle.route(logits.cpu().numpy(), spec.top_k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_router_logits_many_tokens_sampled(act):
    """70,001 tokens (a ragged last tile and block; grids of 1,094 and 4,376
    workgroups along tokens), checked on sampled rows including the last."""
    T, H, E = 70001, 256, 40
    print(f"router many tokens T={T} {act}", flush=True)
    x, w, out = _run(T, H, E, act, seed=550)
    rows = np.random.default_rng(551).choice(T, size=64, replace=False)
    rows = np.concatenate([rows, [0, 1, 16, 63, 64, T - 17, T - 16, T - 1]])
    _check(out.cpu().numpy()[rows], x[rows], w)
