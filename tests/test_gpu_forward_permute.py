"""The permutation and routing that ``ds4moe_forward`` computes, bit-exact
against the oracle, read from forward's workspace (``ds4moe_workspace_region``).

From 256 tokens forward spreads the permutation over 128-token blocks (three
launches: block counts, column scan, bitmap-popcount scatter); below that it
runs the one-workgroup kernel that ``ds4moe_permute`` also runs.  Both must
give the unique stable (expert, token) order.  The cases cover one token (on a
layer shape the batch-1 path does not take), small batches, the first blocked
count, a one-token last block, uniform and Zipf-skewed routing, 8 to 1024
experts, top-k up to 64 (every expert chosen when k = E) and 65,536 tokens.  Where the oracle's O(E^2) rank count over
every token would take minutes (65,536 tokens with 1024 experts), the route
is checked on 512 sampled tokens and the permutation against
``oracle.permute`` of forward's own routing.  ``ds4moe_permute`` (the
one-workgroup kernel) is run on the same routing and must agree too.

The layers are small (hidden 256, expert ffn 128): only the routing matters
here.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import LayerSpec, make_layer, make_x, make_logits

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, weights, to_dev, workspace, ws_tensor  # noqa: E402

CASES = [
    # T, E, k, zipf
    (1, 256, 8, None),        # one token off the batch-1 path
    (2, 8, 2, None),
    (6, 256, 8, None),
    (16, 256, 8, 1.1),
    (31, 64, 64, None),       # k = E: every token takes every expert
    (32, 1024, 64, 1.1),      # the largest E and k
    (33, 256, 8, None),
    (255, 8, 2, None),        # last count on the one-workgroup kernel
    (256, 8, 2, None),        # first blocked count
    (257, 256, 8, None),      # one token in the last block
    (4096, 256, 8, None),     # the prefill routing
    (4096, 256, 8, 1.1),
    (4096, 1024, 8, None),
    (65536, 64, 8, None),
    (65536, 1024, 8, 1.1),
]


@pytest.mark.parametrize("T,E,k,zipf", CASES, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_{'zipf' if c[3] else 'unif'}"
                                                   for c in CASES])
def test_forward_permutation_bitexact(T, E, k, zipf):
    print(f"forward permutation T={T} E={E} k={k} zipf={zipf}", flush=True)
    spec = LayerSpec(256, 128, E, k, 0, "q2k")
    dl = to_dev(make_layer(spec, seed=900 + E, device="cpu"))
    x = make_x(T, spec.hidden, seed=901, dtype="bf16")
    logits = make_logits(T, E, seed=902 + T, zipf_s=zipf)
    cfg = config(spec, algo="auto")
    ws = workspace(cfg, T)
    y = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)
    ds4.forward(cfg, weights(dl), T, x.to(DEV), logits.to(DEV), y, ws)
    torch.cuda.synchronize()
    P = T * k
    gidx = ws_tensor(ws, cfg, T, "topk_idx", torch.int32, (T, k)).cpu().numpy()
    gw = ws_tensor(ws, cfg, T, "topk_w", torch.float32, (T, k)).cpu().numpy().astype(np.float64)
    # route: every token, or 512 sampled ones when the oracle's rank count is too slow
    toks = np.arange(T) if T * E * E <= 5e9 else np.sort(np.random.default_rng(T).choice(T, 512, replace=False))
    ridx, rw = oracle.route(logits.numpy()[toks], k)
    assert np.array_equal(gidx[toks], ridx)
    assert np.max(np.abs(gw[toks] - rw)) <= 2.0 ** -20
    # routing is valid everywhere: k distinct ids per token
    assert gidx.min() >= 0 and gidx.max() < E
    assert all(len(set(r)) == k for r in gidx[:: max(1, T // 4096)].tolist())
    ref = oracle.permute(gidx if toks.size < T else ridx, E)
    got = {n: ws_tensor(ws, cfg, T, n, torch.int32, (m,)).cpu().numpy()
           for n, m in (("offsets", E + 1), ("sorted_pair", P), ("pair_pos", P), ("active", E + 1))}
    n_act = int(ref["active"][0])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["sorted_pair"], ref["sorted_pair"])
    assert np.array_equal(got["pair_pos"], ref["pair_pos"])
    assert np.array_equal(got["active"][:n_act + 1], ref["active"])
    # ds4moe_permute on the same routing (its one-workgroup kernel)
    idx_d = torch.from_numpy(gidx).to(DEV)
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=DEV)
    sp = torch.full((P,), -1, dtype=torch.int32, device=DEV)
    pp = torch.full((P,), -1, dtype=torch.int32, device=DEV)
    act = torch.full((E + 1,), -1, dtype=torch.int32, device=DEV)
    ds4.permute(cfg, T, idx_d, off, sp, pp, act)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), ref["offsets"])
    assert np.array_equal(sp.cpu().numpy(), ref["sorted_pair"])
    assert np.array_equal(pp.cpu().numpy(), ref["pair_pos"])
    assert np.array_equal(act.cpu().numpy()[:n_act + 1], ref["active"])
    print(f"  {n_act} active experts; path {ds4.forward_path(cfg, T)}", flush=True)
