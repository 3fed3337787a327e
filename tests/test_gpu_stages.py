"""GPU parity of the integer and bit-exact stages: route, permute, dequantize,
and the weighted combine, each against the CPU oracle through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden, golden_q2k_block
from synth import LayerSpec, make_layer, make_logits, q2k_encode, mxfp4_encode

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, rowwise_rel_err  # noqa: E402


def _cfg(E, k, H=256, F=128, act="bf16"):
    return config(LayerSpec(H, F, E, k, 0, "q2k"), act=act)


# ------------------------------------------------------------------ route ----
ROUTE_CASES = [
    (16, 8, 2, None), (1, 256, 8, None), (32, 256, 8, 1.1), (4096, 256, 8, None),
    (37, 1024, 64, None), (5, 64, 64, None), (129, 8, 8, None), (3, 1, 1, None),
]


@pytest.mark.parametrize("T,E,k,zipf", ROUTE_CASES)
def test_route_matches_oracle(T, E, k, zipf):
    print(f"route T={T} E={E} k={k} zipf={zipf}", flush=True)
    logits = make_logits(T, E, seed=101, zipf_s=zipf)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    ds4.route(_cfg(E, k), T, logits.to(DEV), idx, w)
    torch.cuda.synchronize()
    ridx, rw = oracle.route(logits.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    gw = w.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gw - rw)) <= 2.0 ** -20
    assert np.all(np.abs(gw.sum(axis=1) - 1.0) <= 1e-6)


def test_route_ties_and_signed_zero():
    rng = np.random.default_rng(7)
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32)
    T, E, k = 200, 16, 5
    logits = torch.from_numpy(vals[rng.integers(0, 5, size=(T, E))])
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ds4.route(_cfg(E, k), T, logits.to(DEV), idx, w)
    torch.cuda.synchronize()
    ridx, rw = oracle.route(logits.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 2.0 ** -20


def test_route_golden_cases():
    for case in load_golden("route_cases.json")["cases"]:
        l = torch.tensor([case["logits"]], dtype=torch.float32)
        E, k = l.shape[1], case["k"]
        idx = torch.empty((1, k), dtype=torch.int32, device=DEV)
        w = torch.empty((1, k), dtype=torch.float32, device=DEV)
        ds4.route(_cfg(E, k), 1, l.to(DEV), idx, w)
        torch.cuda.synchronize()
        assert idx.cpu().numpy()[0].tolist() == case["idx"], case["id"]
        assert np.max(np.abs(w.cpu().numpy()[0] - np.array(case["w"]))) <= 2.0 ** -20, case["id"]


# ---------------------------------------------------------------- permute ----
PERM_CASES = [(16, 8, 2, None), (1, 256, 8, None), (32, 256, 8, 1.1), (4096, 256, 8, None),
              (5000, 8, 2, None), (3000, 1024, 4, None), (1025, 300, 3, 1.1), (1, 1, 1, None)]


@pytest.mark.parametrize("T,E,k,zipf", PERM_CASES)
def test_permute_matches_oracle(T, E, k, zipf):
    print(f"permute T={T} E={E} k={k} zipf={zipf}", flush=True)
    idx, _ = oracle.route(make_logits(T, E, seed=202, zipf_s=zipf).numpy(), k)
    ref = oracle.permute(idx, E)
    P = T * k
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=DEV)
    sp = torch.full((P,), -1, dtype=torch.int32, device=DEV)
    pp = torch.full((P,), -1, dtype=torch.int32, device=DEV)
    act = torch.full((E + 1,), -1, dtype=torch.int32, device=DEV)
    ds4.permute(_cfg(E, k), T, torch.from_numpy(idx.astype(np.int32)).to(DEV), off, sp, pp, act)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), ref["offsets"])
    assert np.array_equal(sp.cpu().numpy(), ref["sorted_pair"])
    assert np.array_equal(pp.cpu().numpy(), ref["pair_pos"])
    n = int(ref["active"][0])
    assert np.array_equal(act.cpu().numpy()[:n + 1], ref["active"])


# ------------------------------------------------------------- dequantize ----
def _dequant(wfmt, data, scales, n):
    f = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    b = torch.zeros((n,), dtype=torch.int16, device=DEV)
    ds4.dequantize(wfmt, data.to(DEV), None if scales is None else scales.to(DEV), n, f, b)
    torch.cuda.synchronize()
    return f.cpu().numpy(), b.cpu().numpy().view(np.uint16)


def _check_bits(f32, bf16, exact):
    ref32 = oracle.fp32_round(exact)
    assert np.array_equal(f32.view(np.uint32), ref32.view(np.uint32))
    assert np.array_equal(bf16, oracle.bf16_bits_from_fp32(ref32))


def test_dequant_q2k_golden_blocks():
    blocks = load_golden("q2k_blocks.json")["blocks"]
    raw = np.frombuffer(b"".join(golden_q2k_block(b) for b in blocks), dtype=np.uint8).copy()
    n = 256 * len(blocks)
    f, b = _dequant("q2k", torch.from_numpy(raw), None, n)
    _check_bits(f, b, oracle.q2k_decode(raw))


def test_dequant_q2k_random_bytes_and_layer():
    rng = np.random.default_rng(3)
    raw = rng.integers(0, 256, size=(4096, 84), dtype=np.uint8)
    raw[:, 81] &= 0x3B
    raw[:, 83] &= 0x3B
    raw = raw.reshape(-1)
    f, b = _dequant("q2k", torch.from_numpy(raw), None, 4096 * 256)
    _check_bits(f, b, oracle.q2k_decode(raw))
    w = torch.from_numpy(rng.standard_normal((512, 256)).astype(np.float32) * 0.02)
    data = q2k_encode(w).reshape(-1)
    f, b = _dequant("q2k", data, None, 512 * 256)
    _check_bits(f, b, oracle.q2k_decode(data.numpy()))


def test_dequant_mxfp4_golden_and_random():
    mx = load_golden("mxfp4_values.json")
    codes = np.array([[int(c["code_byte"], 16)] * 16 for c in mx["cases"] if c["id"] != "M5"], dtype=np.uint8)
    scales = np.array([[int(c["scale"], 16)] for c in mx["cases"] if c["id"] != "M5"], dtype=np.uint8)
    rows = codes.shape[0]
    f, b = _dequant("mxfp4", torch.from_numpy(codes.reshape(-1)), torch.from_numpy(scales.reshape(-1)), rows * 32)
    _check_bits(f, b, oracle.mxfp4_decode_matrix(codes, scales, rows, 32).reshape(-1))
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, size=(64, 128), dtype=np.uint8)
    scales = rng.integers(0, 255, size=(64, 8), dtype=np.uint8)       # every finite scale incl. 0, 1
    f, b = _dequant("mxfp4", torch.from_numpy(codes.reshape(-1)), torch.from_numpy(scales.reshape(-1)), 64 * 256)
    _check_bits(f, b, oracle.mxfp4_decode_matrix(codes, scales, 64, 256).reshape(-1))
    w = torch.from_numpy(rng.standard_normal((64, 256)).astype(np.float32) * 0.02)
    c, s = mxfp4_encode(w)
    f, b = _dequant("mxfp4", c.reshape(-1), s.reshape(-1), 64 * 256)
    _check_bits(f, b, oracle.mxfp4_decode_matrix(c.numpy(), s.numpy(), 64, 256).reshape(-1))


def test_dequant_full_size_expert_sample():
    """One expert matrix of the full-size layer, drawn on the device."""
    L = make_layer(LayerSpec(7168, 2048, 2, 1, 0, "q2k"), device=DEV)
    n = 2048 * 7168
    f, b = _dequant("q2k", L.gate[1], None, n)
    _check_bits(f, b, oracle.q2k_decode(L.routed("gate", 1)[0]))


# ---------------------------------------------------------------- combine ----
@pytest.mark.parametrize("act,tol", [("f32", 1e-5), ("bf16", 2e-2)])
@pytest.mark.parametrize("T,H,E,k,shared", [(16, 256, 8, 2, False), (33, 7168, 256, 8, True), (1, 7168, 256, 8, True)])
def test_combine_matches_oracle(act, tol, T, H, E, k, shared):
    rng = np.random.default_rng(5)
    idx, w = oracle.route(make_logits(T, E, seed=303).numpy(), k)
    perm = oracle.permute(idx, E)
    P = T * k
    dt = torch.float32 if act == "f32" else torch.bfloat16
    eo = torch.from_numpy(rng.standard_normal((P, H)).astype(np.float32)).to(dt)
    so = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(dt) if shared else None
    y = torch.full((T, H), float("nan"), dtype=dt, device=DEV)
    cfg = config(LayerSpec(H, 128, E, k, 128 if shared else 0, "q2k"), act=act)
    ds4.combine(cfg, T, eo.to(DEV), torch.from_numpy(perm["pair_pos"].astype(np.int32)).to(DEV),
                torch.from_numpy(w.astype(np.float32)).to(DEV), None if so is None else so.to(DEV), y)
    torch.cuda.synchronize()
    eo64 = eo.float().numpy().astype(np.float64)
    w32 = w.astype(np.float32).astype(np.float64)      # the weights the kernel was given
    ref = np.stack([oracle.combine(w32[t], eo64[perm["pair_pos"][t * k:(t + 1) * k]],
                                   None if so is None else so[t].float().numpy()) for t in range(T)])
    assert rowwise_rel_err(y.float().cpu().numpy(), ref) <= tol


@pytest.mark.parametrize("k", [2, 8])
def test_combine_skips_invalid_slots(k):
    """pair_pos entries outside [0, T*k) add nothing, on the top-8 path (all
    slot rows requested before the sum) and on the general one: the result
    equals the combine over the valid slots alone."""
    T, H, E = 9, 256, 16
    rng = np.random.default_rng(11 + k)
    idx, w = oracle.route(make_logits(T, E, seed=404 + k).numpy(), k)
    perm = oracle.permute(idx, E)
    P = T * k
    pp = perm["pair_pos"].astype(np.int32).copy()
    bad = rng.choice(P, size=P // 3, replace=False)
    pp[bad[0::2]] = -1
    pp[bad[1::2]] = P + 5
    eo = torch.from_numpy(rng.standard_normal((P, H)).astype(np.float32)).to(torch.bfloat16)
    so = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    cfg = config(LayerSpec(H, 128, E, k, 128, "q2k"), act="bf16")
    ds4.combine(cfg, T, eo.to(DEV), torch.from_numpy(pp).to(DEV), torch.from_numpy(w.astype(np.float32)).to(DEV),
                so.to(DEV), y)
    torch.cuda.synchronize()
    eo64 = eo.float().numpy().astype(np.float64)
    w32 = w.astype(np.float32).astype(np.float64)
    ref = []
    for t in range(T):
        js = [j for j in range(k) if 0 <= pp[t * k + j] < P]
        rows = eo64[pp[[t * k + j for j in js]]] if js else np.zeros((0, H))
        ref.append(oracle.combine(w32[t][js], rows, so[t].float().numpy()))
    assert rowwise_rel_err(y.float().cpu().numpy(), np.stack(ref)) <= 2e-2

