"""GPU parity of the expert FFN and the whole layer against the fp64 oracle.

Tolerance (per-token infinity-norm relative error, max over tokens): 1e-5 in
fp32 mode, 2e-2 in the bf16 path.  Small layers are checked on every token;
full-size layers (7168/2048, 256 experts top-8 + shared) on sampled tokens
that the oracle evaluates one by one, plus whole-output properties.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import LayerSpec, WORKLOADS, make_layer, make_x, make_logits

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, weights, rowwise_rel_err, to_dev, workspace  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _x(T, H, act, seed=11):
    return make_x(T, H, seed=seed, dtype="fp32" if act == "f32" else "bf16")


def _forward(dl, cfg, T, x, logits):
    y = torch.full((T, dl.spec.hidden), float("nan"), dtype=x.dtype, device=DEV)
    ws = workspace(cfg, T)
    ds4.forward(cfg, weights(dl), T, x.to(DEV), logits.to(DEV), y, ws)
    torch.cuda.synchronize()
    return y


def _oracle_y(layer, x, logits, tokens=None):
    r = oracle.forward(layer, x.float().numpy(), logits.numpy(), tokens=tokens)
    toks = sorted(r["y"])
    return toks, np.stack([r["y"][t] for t in toks]), r


# ------------------------------------------------------------ small layers ---
SMALL = [
    ("tiny", LayerSpec(256, 128, 8, 2, 0, "q2k"), 16),
    ("tiny_shared", LayerSpec(256, 128, 8, 2, 128, "q2k"), 16),
    ("mx_tiny", LayerSpec(256, 128, 8, 2, 128, "mxfp4"), 16),
    ("one_expert", LayerSpec(512, 256, 1, 1, 0, "q2k"), 5),
    ("k_eq_E", LayerSpec(256, 256, 4, 4, 0, "q2k"), 3),
    ("ragged", LayerSpec(768, 384, 16, 4, 256, "q2k"), 37),
    ("mx_ragged", LayerSpec(768, 384, 16, 4, 256, "mxfp4"), 37),
    # batch-1 decode shapes (the byte-balanced persistent decode kernels)
    ("d1_q2k", LayerSpec(1024, 256, 16, 4, 256, "q2k"), 1),
    ("d1_q2k_noshared", LayerSpec(2048, 512, 32, 8, 0, "q2k"), 1),
    ("d1_mx", LayerSpec(2048, 512, 16, 4, 512, "mxfp4"), 1),
    ("d1_q2k_wide", LayerSpec(7168, 512, 8, 3, 512, "q2k"), 1),
    # the widest hidden size the boundary accepts: the GEMV launches stage 80 KiB (Q2K) and
    # 64 KiB (MXFP4) of LDS per token, fp32 mode 128 KiB
    ("max_width", LayerSpec(32768, 128, 2, 1, 256, "q2k"), 2),
    ("mx_max_width", LayerSpec(32768, 128, 2, 1, 0, "mxfp4"), 2),
]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("name,spec,T", SMALL, ids=[s[0] for s in SMALL])
def test_forward_small_gemv(name, spec, T, act):
    print(f"forward small {name} T={T} act={act} algo=gemv", flush=True)
    layer = make_layer(spec, seed=20 + len(name), device="cpu")
    dl = to_dev(layer)
    x = _x(T, spec.hidden, act)
    logits = make_logits(T, spec.n_experts, seed=21)
    y = _forward(dl, config(spec, act=act, algo="gemv"), T, x, logits)
    _, ref, _ = _oracle_y(layer, x, logits)
    err = rowwise_rel_err(y.float().cpu().numpy(), ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL[act]


# Batch-1 shapes of the two-launch decode layer (route, expert FFNs, shared
# expert and combine fused; forward with AUTO at T = 1).
T1 = [
    ("t1_q2k", LayerSpec(1024, 1024, 16, 4, 256, "q2k")),
    ("t1_q2k_noshared", LayerSpec(2048, 1024, 32, 8, 0, "q2k")),
    ("t1_q2k_k16", LayerSpec(1024, 1024, 64, 16, 2048, "q2k")),
    # an odd expert count: the router keys end off a 16-byte boundary
    ("t1_q2k_odd_e", LayerSpec(1024, 1024, 33, 4, 256, "q2k")),
    ("t1_mx", LayerSpec(1024, 1024, 16, 4, 512, "mxfp4")),
    ("t1_mx_f2048", LayerSpec(2048, 2048, 64, 6, 256, "mxfp4")),
    # k = 8, ffn 2048, shared ffn 2048: the benchmark layer's proportions, small
    ("t1_q2k_k8", LayerSpec(1024, 2048, 64, 8, 2048, "q2k")),
    ("t1_mx_k8", LayerSpec(2048, 2048, 32, 8, 2048, "mxfp4")),
]


@pytest.mark.parametrize("name,spec", T1, ids=[t[0] for t in T1])
def test_forward_batch1_fused(name, spec):
    path = ds4.forward_path(config(spec, act="bf16", algo="auto"), 1)
    print(f"forward batch-1 {name} path={path}", flush=True)
    assert path == 1
    layer = make_layer(spec, seed=70 + len(name), device="cpu")
    dl = to_dev(layer)
    errs = []
    for draw in range(3):
        x = _x(1, spec.hidden, "bf16", seed=71 + draw)
        logits = make_logits(1, spec.n_experts, seed=72 + draw)
        y = _forward(dl, config(spec, act="bf16", algo="auto"), 1, x, logits)
        _, ref, _ = _oracle_y(layer, x, logits)
        errs.append(rowwise_rel_err(y.float().cpu().numpy(), ref))
    print(f"  err={max(errs):.3e}", flush=True)
    assert max(errs) <= TOL["bf16"]


# Token counts at which forward spreads the permutation over 128-token blocks:
# the most experts (1024, top-8: about two tokens each), the first blocked
# count with one token in the last block, and a few experts with long runs.
BLOCKED = [
    ("many_experts", LayerSpec(256, 128, 1024, 8, 0, "q2k"), 300, "auto", None),
    ("one_token_tail", LayerSpec(256, 128, 3, 2, 128, "q2k"), 257, "auto", None),
    ("zipf_gemv_f32", LayerSpec(256, 128, 40, 6, 128, "mxfp4"), 640, "gemv", 1.2),
]


@pytest.mark.parametrize("name,spec,T,algo,zipf", BLOCKED, ids=[b[0] for b in BLOCKED])
def test_forward_blocked_permutation(name, spec, T, algo, zipf):
    act = "f32" if name.endswith("f32") else "bf16"
    print(f"forward blocked-permute {name} T={T} act={act} algo={algo}", flush=True)
    layer = make_layer(spec, seed=90 + len(name), device="cpu")
    x = _x(T, spec.hidden, act, seed=91)
    logits = make_logits(T, spec.n_experts, seed=92, zipf_s=zipf)
    y = _forward(to_dev(layer), config(spec, act=act, algo=algo), T, x, logits)
    _, ref, _ = _oracle_y(layer, x, logits)
    err = rowwise_rel_err(y.float().cpu().numpy(), ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL[act]


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_expert_ffn_stage_tiny(act):
    """expert_out rows and shared_out against the oracle, inputs from the oracle's own routing."""
    spec = LayerSpec(256, 128, 8, 2, 128, "q2k")
    T = 16
    layer = make_layer(spec, seed=31, device="cpu")
    dl = to_dev(layer)
    x = _x(T, spec.hidden, act)
    idx, _ = oracle.route(make_logits(T, 8, seed=32).numpy(), 2)
    perm = oracle.permute(idx, 8)
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    cfg = config(spec, act=act, algo="gemv")
    eo = torch.full((T * 2, 256), float("nan"), dtype=x.dtype, device=DEV)
    so = torch.full((T, 256), float("nan"), dtype=x.dtype, device=DEV)
    ds4.expert_ffn(cfg, weights(dl), T, x.to(DEV), i32(perm["offsets"]), i32(perm["sorted_pair"]),
                   i32(perm["active"]), eo, so, workspace(cfg, T))
    torch.cuda.synchronize()
    o, _ = oracle.expert_outputs(layer, x.float().numpy(), idx)
    ref_eo = np.stack([o[(int(p) // 2, int(p) % 2)] for p in perm["sorted_pair"]])
    assert rowwise_rel_err(eo.float().cpu().numpy(), ref_eo) <= TOL[act]
    s = oracle.shared_outputs(layer, x.float().numpy())
    assert rowwise_rel_err(so.float().cpu().numpy(), np.stack([s[t] for t in range(T)])) <= TOL[act]


def test_forward_deterministic_and_poison_free():
    spec = LayerSpec(768, 384, 16, 4, 256, "q2k")
    T = 37
    dl = to_dev(make_layer(spec, seed=41, device="cpu"))
    x = _x(T, spec.hidden, "bf16")
    logits = make_logits(T, 16, seed=42)
    cfg = config(spec, algo="gemv")
    y1 = _forward(dl, cfg, T, x, logits)
    y2 = _forward(dl, cfg, T, x, logits)
    assert torch.isfinite(y1.float()).all()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------------- full-size layers ---
@pytest.fixture(scope="module")
def q2k_layer():
    return make_layer(WORKLOADS["decode"]["spec"], seed=5150, device=DEV)


@pytest.fixture(scope="module")
def mx_layer():
    return make_layer(WORKLOADS["mxfp4_decode"]["spec"], seed=5151, device=DEV)


@pytest.mark.parametrize("algo", ["auto", "gemv"])
def test_decode_full_size(q2k_layer, algo):
    """Batch-1 decode, 7168/2048, 256 experts top-8 + bf16 shared expert."""
    print(f"decode full size algo={algo}", flush=True)
    spec = q2k_layer.spec
    x = _x(1, spec.hidden, "bf16", seed=12)
    logits = make_logits(1, spec.n_experts, seed=13)
    y = _forward(q2k_layer, config(spec, algo=algo), 1, x, logits)
    _, ref, _ = _oracle_y(q2k_layer, x, logits)
    err = rowwise_rel_err(y.float().cpu().numpy(), ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_decode_full_size_fp32_mode(q2k_layer):
    spec = q2k_layer.spec
    x = _x(1, spec.hidden, "f32", seed=14)
    logits = make_logits(1, spec.n_experts, seed=15)
    y = _forward(q2k_layer, config(spec, act="f32"), 1, x, logits)
    _, ref, _ = _oracle_y(q2k_layer, x, logits)
    err = rowwise_rel_err(y.cpu().numpy(), ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL["f32"]


@pytest.mark.parametrize("algo", ["auto", "gemv"])
def test_mxfp4_decode_full_size(mx_layer, algo):
    print(f"mxfp4 decode full size algo={algo}", flush=True)
    spec = mx_layer.spec
    x = _x(1, spec.hidden, "bf16", seed=18)
    logits = make_logits(1, spec.n_experts, seed=19)
    y = _forward(mx_layer, config(spec, algo=algo), 1, x, logits)
    _, ref, _ = _oracle_y(mx_layer, x, logits)
    err = rowwise_rel_err(y.float().cpu().numpy(), ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


# All-equal router logits: every tie goes to the lower index, so each token
# takes experts 0 .. k-1 with weight 1/k; with all-zero routed blocks (d = dmin
# = 0) every routed output is +0 and y is the shared expert alone.
DEGENERATE = [
    ("batch1", LayerSpec(1024, 1024, 16, 4, 256, "q2k"), 1, "auto"),
    ("gemv", LayerSpec(512, 256, 16, 4, 256, "q2k"), 4, "auto"),
    ("grouped", LayerSpec(512, 256, 16, 4, 256, "q2k"), 40, "auto"),
]


@pytest.mark.parametrize("name,spec,T,algo", DEGENERATE, ids=[d[0] for d in DEGENERATE])
def test_tied_logits_and_zero_routed_blocks(name, spec, T, algo):
    print(f"degenerate {name} T={T}", flush=True)
    layer = make_layer(spec, seed=90 + T, device="cpu")
    x = _x(T, spec.hidden, "bf16", seed=91)
    logits = torch.full((T, spec.n_experts), 0.25, dtype=torch.float32)
    # tied logits, real weights: the oracle's routing (experts 0..k-1, 1/k)
    _, ref, r = _oracle_y(layer, x, logits)
    assert (r["idx"] == np.arange(spec.top_k)[None, :]).all()
    y = _forward(to_dev(layer), config(spec, algo=algo), T, x, logits)
    assert rowwise_rel_err(y.float().cpu().numpy(), ref) <= TOL["bf16"]
    # zero routed blocks: the shared expert alone
    zl = layer.clone()
    for f in ("gate", "up", "down"):
        getattr(zl, f).zero_()
    _, zref, zr = _oracle_y(zl, x, logits)
    assert all(np.all(zr["o"][p] == 0.0) for p in zr["o"])
    yz = _forward(to_dev(zl), config(spec, algo=algo), T, x, logits)
    assert rowwise_rel_err(yz.float().cpu().numpy(), zref) <= TOL["bf16"]
    assert np.allclose(zref, np.stack([zr["s"][t] for t in range(T)]), rtol=0, atol=0)
