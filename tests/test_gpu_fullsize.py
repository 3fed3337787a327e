"""GPU parity of the full-size layers (7168/2048, 256 experts top-8, bf16
shared expert 2048) against the fp64 oracle, in the launch configuration the
benchmark times.

Every check reads what ``ds4moe_forward`` itself produced:
  * the route (expert ids bit-exact, weights within 2^-20) and the
    permutation (offsets, sorted_pair, pair_pos, active: bit-exact), read from
    forward's workspace; at 256 tokens and above forward computes the
    permutation with its blocked kernels, so this checks those;
  * y on every token of the hottest and of the coldest active expert plus 64
    seeded random tokens (4096-token prefill), or on every token (32-token
    batched decode, 2..16-token batches), per-token infinity-norm relative
    error <= 2e-2;
  * the expert_out rows of the hottest and the coldest expert (prefill),
    against the oracle's per-pair outputs, same bar.

The oracle evaluates the sampled tokens' expert pairs per pair (its
definition), with disjoint expert sets on threads (``helpers.oracle_pairs``).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_layer, make_x, make_logits

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, weights, rowwise_rel_err, workspace, ws_tensor, oracle_y  # noqa: E402

TOL = 2e-2


def _run(layer, T, algo, mma, x, logits):
    spec = layer.spec
    cfg = config(spec, algo=algo, mma=mma)
    ws = workspace(cfg, T)
    y = torch.full((T, spec.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds4.forward(cfg, weights(layer), T, x.to(DEV), logits.to(DEV), y, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    return cfg, ws, y


def _check_routing(cfg, ws, T, spec, logits, perm_too=True):
    """Route and (when forward made one) the permutation, bit-exact."""
    k, E = spec.top_k, spec.n_experts
    ridx, rw = oracle.route(logits.numpy(), k)
    gidx = ws_tensor(ws, cfg, T, "topk_idx", torch.int32, (T, k)).cpu().numpy()
    gw = ws_tensor(ws, cfg, T, "topk_w", torch.float32, (T, k)).cpu().numpy().astype(np.float64)
    assert np.array_equal(gidx, ridx)
    assert np.max(np.abs(gw - rw)) <= 2.0 ** -20
    if perm_too:
        ref = oracle.permute(ridx, E)
        for name, n in (("offsets", E + 1), ("sorted_pair", T * k), ("pair_pos", T * k)):
            got = ws_tensor(ws, cfg, T, name, torch.int32, (n,)).cpu().numpy()
            assert np.array_equal(got, ref[name]), name
        act = ws_tensor(ws, cfg, T, "active", torch.int32, (E + 1,)).cpu().numpy()
        n_act = int(ref["active"][0])
        assert np.array_equal(act[:n_act + 1], ref["active"])
        return ridx, ref
    return ridx, None


def _sample(idx, E, T, seed):
    """Every token of the hottest and of the coldest active expert (lowest id
    on ties), plus 64 seeded random tokens."""
    counts = np.bincount(idx.ravel(), minlength=E)
    hot = int(np.argmax(counts))
    act = np.nonzero(counts)[0]
    cold = int(act[np.argmin(counts[act])])
    toks = set(np.nonzero((idx == hot).any(axis=1))[0].tolist())
    toks |= set(np.nonzero((idx == cold).any(axis=1))[0].tolist())
    toks |= set(np.random.default_rng(seed).choice(T, 64, replace=False).tolist())
    return sorted(toks), hot, cold, counts


@pytest.fixture(scope="module")
def q2k_layer():
    return make_layer(WORKLOADS["prefill"]["spec"], seed=6150, device=DEV)


@pytest.fixture(scope="module")
def mx_layer():
    return make_layer(WORKLOADS["mxfp4_prefill"]["spec"], seed=6151, device=DEV)


PREFILL = [("q2k", "bf16"), ("mxfp4", "bf16"), ("mxfp4", "fp8")]


@pytest.mark.parametrize("fmt,mma", PREFILL, ids=[f"{f}_{m}" for f, m in PREFILL])
def test_prefill_full_size(fmt, mma, q2k_layer, mx_layer):
    """4096 tokens, uniform routing, AUTO (the grouped GEMM, blocked permutation)."""
    layer = q2k_layer if fmt == "q2k" else mx_layer
    spec, T, k = layer.spec, 4096, layer.spec.top_k
    seed = {"q2k": 7, "mxfp4": 9}[fmt] + (100 if mma == "fp8" else 0)
    print(f"prefill full size {fmt} mma={mma}", flush=True)
    x = make_x(T, spec.hidden, seed=100 + seed, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=200 + seed)
    cfg, ws, y = _run(layer, T, "auto", mma, x, logits)
    assert ds4.forward_path(cfg, T) == 2
    idx, perm = _check_routing(cfg, ws, T, spec, logits)
    toks, hot, cold, counts = _sample(idx, spec.n_experts, T, seed)
    print(f"  hottest expert {hot} ({counts[hot]} tokens), coldest {cold} ({counts[cold]}), "
          f"{len(toks)} tokens sampled", flush=True)
    yref, r = oracle_y(layer, x.float().numpy(), logits.numpy(), toks, mx8=(mma == "fp8"))
    err = rowwise_rel_err(y.float().cpu().numpy()[toks], yref)
    eo = ws_tensor(ws, cfg, T, "expert_out", torch.bfloat16, (T * k, spec.hidden)).float().cpu().numpy()
    errs = {}
    for e in (hot, cold):
        rows = np.arange(perm["offsets"][e], perm["offsets"][e + 1])
        pairs = perm["sorted_pair"][rows]
        ref = np.stack([r["o"][(int(p) // k, int(p) % k)] for p in pairs])
        errs[e] = rowwise_rel_err(eo[rows], ref)
    print(f"  y err {err:.3e}; expert_out err hot {errs[hot]:.3e} cold {errs[cold]:.3e}", flush=True)
    assert err <= TOL
    assert max(errs.values()) <= TOL


@pytest.mark.parametrize("algo", ["auto", "gemv", "grouped"])
def test_batched_decode_zipf_all_tokens(q2k_layer, algo):
    """32 tokens, Zipf(1.1)-skewed routing: every token against the oracle
    (AUTO runs the grouped GEMM's small-batch layout)."""
    spec, T = q2k_layer.spec, 32
    print(f"batched decode 32 Zipf algo={algo}", flush=True)
    x = make_x(T, spec.hidden, seed=108, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=208, zipf_s=1.1)
    cfg, ws, y = _run(q2k_layer, T, algo, "bf16", x, logits)
    _check_routing(cfg, ws, T, spec, logits)
    toks = list(range(T))
    yref, r = oracle_y(q2k_layer, x.float().numpy(), logits.numpy(), toks)
    n_act = len({int(e) for e in r["idx"].ravel()})
    err = rowwise_rel_err(y.float().cpu().numpy(), yref)
    print(f"  {n_act} active experts, err {err:.3e}", flush=True)
    assert err <= TOL


# Small batches through the GEMV / grouped crossover: 1 + 5 speculative draft
# tokens (6), and 2..16 concurrent sessions.  The oracle's outputs for the 16
# tokens are computed once: a token's output depends only on its own x and
# logits, so the first T tokens' references serve every T.
SMALL_T = [2, 6, 8, 16]


@pytest.fixture(scope="module")
def small_batch_ref(q2k_layer):
    spec = q2k_layer.spec
    x = make_x(16, spec.hidden, seed=109, dtype="bf16")
    logits = make_logits(16, spec.n_experts, seed=209)
    yref, r = oracle_y(q2k_layer, x.float().numpy(), logits.numpy(), list(range(16)))
    return x, logits, yref


@pytest.mark.parametrize("algo", ["auto", "gemv", "grouped"])
@pytest.mark.parametrize("T", SMALL_T)
def test_small_batch_full_size(q2k_layer, small_batch_ref, T, algo):
    x16, logits16, yref = small_batch_ref
    spec = q2k_layer.spec
    print(f"small batch T={T} algo={algo}", flush=True)
    x, logits = x16[:T].contiguous(), logits16[:T].contiguous()
    cfg, ws, y = _run(q2k_layer, T, algo, "bf16", x, logits)
    _check_routing(cfg, ws, T, spec, logits)
    err = rowwise_rel_err(y.float().cpu().numpy(), yref[:T])
    print(f"  path {ds4.forward_path(cfg, T)} err {err:.3e}", flush=True)
    assert err <= TOL


@pytest.fixture(scope="module")
def mx_small_ref(mx_layer):
    spec = mx_layer.spec
    x = make_x(6, spec.hidden, seed=110, dtype="bf16")
    logits = make_logits(6, spec.n_experts, seed=210)
    yref, r = oracle_y(mx_layer, x.float().numpy(), logits.numpy(), list(range(6)))
    return x, logits, yref


@pytest.mark.parametrize("T", [2, 6])
def test_small_batch_gemv_mxfp4_full_size(mx_layer, mx_small_ref, T):
    """MXFP4 experts through the GEMV launches: at 6 tokens the down items
    take twice the passes (48 routed pairs keep the item count above 1024),
    at 2 tokens they do not (16 pairs); every token against the oracle."""
    x6, logits6, yref = mx_small_ref
    spec = mx_layer.spec
    print(f"mxfp4 small batch T={T} gemv", flush=True)
    x, logits = x6[:T].contiguous(), logits6[:T].contiguous()
    cfg, ws, y = _run(mx_layer, T, "gemv", "bf16", x, logits)
    _check_routing(cfg, ws, T, spec, logits)
    err = rowwise_rel_err(y.float().cpu().numpy(), yref[:T])
    print(f"  path {ds4.forward_path(cfg, T)} err {err:.3e}", flush=True)
    assert ds4.forward_path(cfg, T) == 0
    assert err <= TOL


def test_decode_batch1_routing_kept(q2k_layer):
    """The batch-1 launches keep the route in the workspace: bit-exact."""
    spec = q2k_layer.spec
    x = make_x(1, spec.hidden, seed=110, dtype="bf16")
    logits = make_logits(1, spec.n_experts, seed=210)
    cfg, ws, y = _run(q2k_layer, 1, "auto", "bf16", x, logits)
    assert ds4.forward_path(cfg, 1) == 1
    _check_routing(cfg, ws, 1, spec, logits, perm_too=False)
