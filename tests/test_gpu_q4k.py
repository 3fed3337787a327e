"""GPU parity of the Q4K-style 4-bit routed experts against the fp64 oracle.

- ds4moe_dequantize: fp32 and bf16 bit patterns equal to the oracle's exact
  weight rounded once to fp32 (then that to bf16), on the hand-worked blocks
  and on random bytes;
- the layer in fp32 mode (<= 1e-5) and on the bf16 path (<= 2e-2, per-token
  infinity-norm relative error) through every kernel family that takes Q4K
  experts, on small layers (every token) and on the full-size 7168/2048,
  256-expert top-8 layer with its bf16 shared expert (decode on every token,
  prefill on the hottest and coldest expert's tokens plus 64 random ones).
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden
from synth import LayerSpec, WORKLOADS, make_layer, make_x, make_logits

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, weights, rowwise_rel_err, to_dev, workspace, oracle_y  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _golden_blocks():
    """(codes [n][128], params [n][20]) of the hand-worked blocks."""
    out_c, out_p = [], []
    for spec in load_golden("q4k_blocks.json")["blocks"]:
        if spec.get("codes") == "staircase":
            codes = [(2 * j) % 16 | (((2 * j + 1) % 16) << 4) for j in range(128)]
        else:
            head = [int(h, 16) for h in spec["codes_head"]]
            codes = head + [int(spec["codes_fill"], 16)] * (128 - len(head))
        sc, i = [], 0
        lst = spec["scales"]
        while i < len(lst):
            v = int(lst[i], 16)
            if i + 1 < len(lst) and isinstance(lst[i + 1], int):
                sc += [v] * lst[i + 1]
                i += 2
            else:
                sc.append(v)
                i += 1
        d, dm = int(spec["d"], 16), int(spec["dmin"], 16)
        out_c.append(codes)
        out_p.append(sc + [d & 0xFF, d >> 8, dm & 0xFF, dm >> 8])
    return np.array(out_c, dtype=np.uint8), np.array(out_p, dtype=np.uint8)


def _dequant(codes, params):
    n = codes.size * 2
    cd = torch.from_numpy(codes.reshape(-1)).to(DEV)
    pd = torch.from_numpy(params.reshape(-1)).to(DEV)
    f32 = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    b16 = torch.full((n,), -1, dtype=torch.int16, device=DEV)
    ds4.dequantize("q4k", cd, pd, n, out_f32=f32, out_bf16=b16)
    torch.cuda.synchronize()
    return f32.cpu().numpy(), b16.cpu().numpy().view(np.uint16)


def test_dequant_q4k_bitexact():
    gc, gp = _golden_blocks()
    rng = np.random.default_rng(31)
    rc = rng.integers(0, 256, size=(2000, 128), dtype=np.uint8)
    rp = rng.integers(0, 256, size=(2000, 20), dtype=np.uint8)
    rp[:, 17] &= 0xBB                 # finite d and dmin of both signs (exponent < 31)
    rp[:, 19] &= 0xBB
    codes = np.concatenate([gc, rc])
    params = np.concatenate([gp, rp])
    nb = codes.shape[0]
    exact = oracle.q4k_decode_matrix(codes.reshape(-1), params.reshape(-1), nb, 256).reshape(-1)
    w32 = oracle.fp32_round(exact)
    f32, b16 = _dequant(codes, params)
    assert np.array_equal(f32.view(np.uint32), w32.view(np.uint32))
    assert np.array_equal(b16, oracle.bf16_bits_from_fp32(w32))


def test_dequant_q4k_matrix_of_a_layer():
    """Every weight of one expert's gate matrix of an encoded layer (the
    fixture's bytes), bit for bit."""
    spec = LayerSpec(1024, 512, 2, 1, 0, "q4k")
    layer = make_layer(spec, seed=32, device="cpu")
    c, p = layer.routed("gate", 1)
    W = oracle.q4k_decode_matrix(c, p, 512, 1024)
    f32, _ = _dequant(c, p)
    assert np.array_equal(f32.view(np.uint32), oracle.fp32_round(W).reshape(-1).view(np.uint32))


def _forward(dl, cfg, T, x, logits):
    y = torch.full((T, dl.spec.hidden), float("nan"), dtype=x.dtype, device=DEV)
    ds4.forward(cfg, weights(dl), T, x.to(DEV), logits.to(DEV), y, workspace(cfg, T))
    torch.cuda.synchronize()
    return y


SMALL = [
    # name, spec, T
    ("tiny", LayerSpec(256, 256, 8, 2, 0, "q4k"), 16),
    ("ragged", LayerSpec(768, 512, 16, 4, 256, "q4k"), 37),
    ("one_expert", LayerSpec(512, 256, 1, 1, 0, "q4k"), 5),
    ("k_eq_E", LayerSpec(256, 256, 4, 4, 128, "q4k"), 3),
    ("decode", LayerSpec(1024, 1024, 16, 4, 256, "q4k"), 1),
    ("decode_k8", LayerSpec(2048, 2048, 32, 8, 2048, "q4k"), 1),
    ("wide", LayerSpec(2048, 2048, 8, 2, 2048, "q4k"), 40),
    ("split", LayerSpec(512, 256, 4, 2, 256, "q4k"), 500),
    ("max_width", LayerSpec(32768, 256, 2, 1, 256, "q4k"), 2),   # 72 KiB of staged LDS per token
]


@pytest.mark.parametrize("algo", ["auto", "gemv", "grouped"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("name,spec,T", SMALL, ids=[s[0] for s in SMALL])
def test_q4k_forward_small(name, spec, T, act, algo):
    if act == "f32" and algo == "grouped":
        pytest.skip("fp32 mode runs the GEMV kernels only")
    cfg = config(spec, act=act, algo=algo)
    if algo == "grouped" and ds4.forward_path(cfg, T) != 2:
        pytest.skip("this shape does not run on the grouped GEMM")
    print(f"q4k forward {name} T={T} act={act} algo={algo} path={ds4.forward_path(cfg, T)}", flush=True)
    layer = make_layer(spec, seed=40 + len(name), device="cpu")
    dl = to_dev(layer)
    x = make_x(T, spec.hidden, seed=41, dtype="fp32" if act == "f32" else "bf16")
    logits = make_logits(T, spec.n_experts, seed=42)
    y = _forward(dl, cfg, T, x, logits)
    r = oracle.forward(layer, x.float().numpy(), logits.numpy())
    ref = np.stack([r["y"][t] for t in range(T)])
    err = rowwise_rel_err(y.float().cpu().numpy(), ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL[act]


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_q4k_expert_ffn_stage(act):
    """expert_out rows and shared_out against the oracle, routing from the oracle."""
    spec = LayerSpec(512, 256, 8, 2, 256, "q4k")
    T = 24
    layer = make_layer(spec, seed=43, device="cpu")
    dl = to_dev(layer)
    x = make_x(T, spec.hidden, seed=44, dtype="fp32" if act == "f32" else "bf16")
    idx, _ = oracle.route(make_logits(T, 8, seed=45).numpy(), 2)
    perm = oracle.permute(idx, 8)
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    cfg = config(spec, act=act, algo="gemv")
    eo = torch.full((T * 2, 512), float("nan"), dtype=x.dtype, device=DEV)
    so = torch.full((T, 512), float("nan"), dtype=x.dtype, device=DEV)
    ds4.expert_ffn(cfg, weights(dl), T, x.to(DEV), i32(perm["offsets"]), i32(perm["sorted_pair"]),
                   i32(perm["active"]), eo, so, workspace(cfg, T))
    torch.cuda.synchronize()
    o, _ = oracle.expert_outputs(layer, x.float().numpy(), idx)
    ref_eo = np.stack([o[(int(p) // 2, int(p) % 2)] for p in perm["sorted_pair"]])
    assert rowwise_rel_err(eo.float().cpu().numpy(), ref_eo) <= TOL[act]
    s = oracle.shared_outputs(layer, x.float().numpy())
    assert rowwise_rel_err(so.float().cpu().numpy(), np.stack([s[t] for t in range(T)])) <= TOL[act]


def test_q4k_zero_blocks_leave_shared_only():
    spec = LayerSpec(512, 256, 16, 4, 256, "q4k")
    T = 9
    layer = make_layer(spec, seed=46, device="cpu")
    zl = layer.clone()
    for f in ("gate", "up", "down", "gate_scales", "up_scales", "down_scales"):
        getattr(zl, f).zero_()
    x = make_x(T, spec.hidden, seed=47, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=48)
    r = oracle.forward(zl, x.float().numpy(), logits.numpy())
    ref = np.stack([r["s"][t] for t in range(T)])
    for algo in ("auto", "gemv"):
        y = _forward(to_dev(zl), config(spec, algo=algo), T, x, logits)
        assert rowwise_rel_err(y.float().cpu().numpy(), ref) <= TOL["bf16"]


# ------------------------------------------------------------- full size ---
@pytest.fixture(scope="module")
def q4_layer():
    return make_layer(LayerSpec(7168, 2048, 256, 8, 2048, "q4k"), seed=8150, device=DEV)


@pytest.mark.parametrize("algo", ["auto", "gemv"])
def test_q4k_decode_full_size(q4_layer, algo):
    spec = q4_layer.spec
    cfg = config(spec, algo=algo)
    print(f"q4k decode full size algo={algo} path={ds4.forward_path(cfg, 1)}", flush=True)
    # AUTO takes the two-launch batch-1 path at this shape
    assert ds4.forward_path(cfg, 1) == (1 if algo == "auto" else 0)
    errs = []
    for draw in range(3):
        x = make_x(1, spec.hidden, seed=50 + draw, dtype="bf16")
        logits = make_logits(1, spec.n_experts, seed=60 + draw)
        y = _forward(q4_layer, cfg, 1, x, logits)
        yref, _ = oracle_y(q4_layer, x.float().numpy(), logits.numpy(), [0])
        errs.append(rowwise_rel_err(y.float().cpu().numpy(), yref))
    print(f"  err={max(errs):.3e}", flush=True)
    assert max(errs) <= TOL["bf16"]


@pytest.mark.parametrize("T", [2, 6])
def test_q4k_small_batch_gemv_full_size(q4_layer, T):
    """Q4K experts through the GEMV launches at 2 and 6 tokens (at 6 the down
    items take twice the passes, at 2 they do not): every token."""
    spec = q4_layer.spec
    x = make_x(T, spec.hidden, seed=80 + T, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=90 + T)
    cfg = config(spec, algo="gemv")
    print(f"q4k small batch T={T} gemv path={ds4.forward_path(cfg, T)}", flush=True)
    assert ds4.forward_path(cfg, T) == 0
    y = _forward(q4_layer, cfg, T, x, logits)
    yref, _ = oracle_y(q4_layer, x.float().numpy(), logits.numpy(), list(range(T)))
    err = rowwise_rel_err(y.float().cpu().numpy(), yref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_q4k_batched_decode_full_size(q4_layer):
    """32 Zipf-routed tokens through AUTO, every token."""
    spec, T = q4_layer.spec, 32
    x = make_x(T, spec.hidden, seed=70, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=71, zipf_s=1.1)
    cfg = config(spec, algo="auto")
    print(f"q4k batched decode path={ds4.forward_path(cfg, T)}", flush=True)
    y = _forward(q4_layer, cfg, T, x, logits)
    yref, _ = oracle_y(q4_layer, x.float().numpy(), logits.numpy(), list(range(T)))
    err = rowwise_rel_err(y.float().cpu().numpy(), yref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_q4k_prefill_full_size(q4_layer):
    """4096 tokens, uniform routing, AUTO: the hottest and the coldest
    expert's tokens plus 64 random ones."""
    spec, T = q4_layer.spec, 4096
    x = make_x(T, spec.hidden, seed=72, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=73)
    cfg = config(spec, algo="auto")
    print(f"q4k prefill full size path={ds4.forward_path(cfg, T)}", flush=True)
    y = _forward(q4_layer, cfg, T, x, logits)
    assert torch.isfinite(y.float()).all()
    idx, _ = oracle.route(logits.numpy(), spec.top_k)
    counts = np.bincount(idx.ravel(), minlength=spec.n_experts)
    hot, cold = int(np.argmax(counts)), int(np.argmin(counts))
    toks = set(np.nonzero((idx == hot).any(axis=1))[0].tolist()) | set(np.nonzero((idx == cold).any(axis=1))[0].tolist())
    toks |= set(np.random.default_rng(74).choice(T, 64, replace=False).tolist())
    toks = sorted(toks)
    yref, _ = oracle_y(q4_layer, x.float().numpy(), logits.numpy(), toks)
    err = rowwise_rel_err(y.float().cpu().numpy()[toks], yref)
    print(f"  {len(toks)} tokens, err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


Q4_T1 = [
    ("t1_q4k_k8", LayerSpec(2048, 2048, 32, 8, 2048, "q4k")),
    ("t1_q4k_noshared", LayerSpec(1024, 2048, 16, 4, 0, "q4k")),
    ("t1_q4k_k12", LayerSpec(1024, 2048, 64, 12, 1024, "q4k")),
    ("t1_q4k_h4096", LayerSpec(4096, 2048, 64, 8, 2048, "q4k")),
]


@pytest.mark.parametrize("name,spec", Q4_T1, ids=[t[0] for t in Q4_T1])
def test_q4k_batch1_fused(name, spec):
    """The two-launch batch-1 layer on Q4K experts (rows up to 7168 wide,
    ffn 2048), three router draws each."""
    cfg = config(spec, algo="auto")
    assert ds4.forward_path(cfg, 1) == 1
    layer = make_layer(spec, seed=80 + len(name), device="cpu")
    dl = to_dev(layer)
    errs = []
    for draw in range(3):
        x = make_x(1, spec.hidden, seed=81 + draw, dtype="bf16")
        logits = make_logits(1, spec.n_experts, seed=82 + draw)
        y = _forward(dl, cfg, 1, x, logits)
        r = oracle.forward(layer, x.float().numpy(), logits.numpy())
        errs.append(rowwise_rel_err(y.float().cpu().numpy(), r["y"][0][None, :]))
    print(f"q4k batch-1 {name}: err={max(errs):.3e}", flush=True)
    assert max(errs) <= TOL["bf16"]
