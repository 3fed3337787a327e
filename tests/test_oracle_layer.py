"""Pins for the oracle's routing, permutation, FFN and combine (CPU only).

Checked against hand-worked cases (tests/golden), brute force with Python's
``sorted`` on tiny inputs, closed forms (scipy's softmax / expit), special
cases that reduce to a dense FFN, and invariants.
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy.special import expit, softmax

import oracle
from conftest import load_golden
from synth import LayerSpec, make_layer, make_x, make_logits, WORKLOADS


# ------------------------------------------------------------------ route ----
ROUTE = load_golden("route_cases.json")["cases"]


@pytest.mark.parametrize("case", ROUTE, ids=[c["id"] for c in ROUTE])
def test_route_golden(case):
    l = np.array([case["logits"]], dtype=np.float32)
    idx, w = oracle.route(l, case["k"])
    assert idx[0].tolist() == case["idx"]
    assert np.allclose(w[0], case["w"], rtol=0, atol=1e-15)


def _brute_route(row, k):
    keys = sorted(range(len(row)), key=lambda i: (-float(row[i]), i))
    return keys[:k]


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 9).flatmap(lambda E: st.tuples(
    st.lists(st.sampled_from([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 2.0]), min_size=E, max_size=E),
    st.integers(1, E))))
def test_route_brute_force_with_ties(args):
    row, k = args
    l = np.array([row], dtype=np.float32)
    idx, w = oracle.route(l, k)
    assert idx[0].tolist() == _brute_route(row, k)
    assert np.all(w > 0) and abs(w.sum() - 1.0) < 1e-15
    # equal logits carry equal weights
    sel = np.array(row)[idx[0]]
    for a in range(k):
        for b in range(k):
            if sel[a] == sel[b]:
                assert w[0, a] == w[0, b]


def test_route_literal_chain_agrees():
    l = make_logits(64, 256, seed=11).numpy()
    idx, w = oracle.route(l, 8)
    idx2, w2 = oracle.route_softmax_chain(l, 8)
    assert np.array_equal(idx, idx2)
    assert np.max(np.abs(w - w2)) < 1e-15


def test_route_k_equals_E_is_full_softmax():
    l = make_logits(5, 8, seed=12).numpy()
    idx, w = oracle.route(l, 8)
    p = softmax(l.astype(np.float64), axis=1)
    for t in range(5):
        assert sorted(idx[t].tolist()) == list(range(8))
        assert np.allclose(w[t], p[t, idx[t]], rtol=1e-14, atol=0)


def test_route_invariants_zipf():
    l = make_logits(32, 256, seed=13, zipf_s=1.1).numpy()
    idx, w = oracle.route(l, 8)
    for t in range(32):
        assert len(set(idx[t].tolist())) == 8
        assert np.all((idx[t] >= 0) & (idx[t] < 256))
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)
    # the bias concentrates load: fewer distinct experts than uniform would give
    assert len(np.unique(idx)) < 200


# ---------------------------------------------------------------- permute ----
PERM = load_golden("permute_cases.json")["cases"]


@pytest.mark.parametrize("case", PERM, ids=[c["id"] for c in PERM])
def test_permute_golden(case):
    r = oracle.permute(np.array(case["idx"]), case["E"])
    for key in ("counts", "offsets", "sorted_pair", "pair_pos", "active"):
        assert r[key].tolist() == case[key], key


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 12).flatmap(lambda E: st.tuples(
    st.just(E), st.integers(1, E).flatmap(lambda k: st.tuples(
        st.just(k), st.integers(1, 9).flatmap(lambda T: st.lists(
            st.permutations(list(range(E))).map(lambda p: p[:k]), min_size=T, max_size=T)))))))
def test_permute_brute_force(args):
    E, (k, rows) = args
    idx = np.array(rows)
    T = idx.shape[0]
    r = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    ref = sorted(range(T * k), key=lambda p: (flat[p], p // k))
    assert r["sorted_pair"].tolist() == ref
    assert r["counts"].sum() == T * k
    assert np.all(np.diff(r["offsets"]) >= 0) and r["offsets"][-1] == T * k
    assert np.array_equal(r["pair_pos"][r["sorted_pair"]], np.arange(T * k))
    act = r["active"]
    assert act[0] == len(set(flat.tolist())) and act[1:].tolist() == sorted(set(flat.tolist()))
    for e in range(E):
        seg = r["sorted_pair"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg // k) > 0)


# -------------------------------------------------------------------- FFN ----
def test_silu_values():
    assert oracle.silu(1.0) == 0.7310585786300049
    assert oracle.silu(0.0) == 0.0
    g = np.linspace(-30, 30, 1001)
    assert np.allclose(oracle.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)
    assert oracle.silu(-1000.0) == 0.0


def _tiny_layer(spec, seed=5):
    return make_layer(spec, seed=seed, device="cpu")


def test_single_expert_is_dense_ffn():
    """E = 1, k = 1, no shared expert: the layer is one dense SwiGLU FFN."""
    spec = LayerSpec(256, 128, 1, 1, 0, "q2k")
    L = _tiny_layer(spec)
    x = make_x(6, 256, seed=7, dtype="fp32").numpy().astype(np.float64)
    logits = np.zeros((6, 1), dtype=np.float32)
    r = oracle.forward(L, x, logits)
    Wg, Wu, Wd = (oracle.decode_routed(L, n, 0) for n in ("gate", "up", "down"))
    G = x @ Wg.T
    ref = (G * expit(G) * (x @ Wu.T)) @ Wd.T
    got = np.stack([r["y"][t] for t in range(6)])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_tiny_matches_dense_mixture():
    """The tiny workload: per-token routed evaluation equals the dense mixture
    over all experts with the scattered gate weights."""
    wl = WORKLOADS["tiny"]
    L = _tiny_layer(wl["spec"])
    x = make_x(wl["T"], 256, dtype="fp32").numpy()
    logits = make_logits(wl["T"], 8).numpy()
    r = oracle.forward(L, x, logits)
    Y = oracle.dense_mixture(L, x, logits)
    got = np.stack([r["y"][t] for t in range(wl["T"])])
    assert np.allclose(got, Y, rtol=1e-12, atol=1e-14)


def test_k_equals_E_is_softmax_mixture():
    spec = LayerSpec(256, 128, 4, 4, 0, "q2k")
    L = _tiny_layer(spec)
    x = make_x(3, 256, seed=8, dtype="fp32").numpy().astype(np.float64)
    logits = make_logits(3, 4, seed=9).numpy()
    p = softmax(logits.astype(np.float64), axis=1)
    ref = np.zeros((3, 256))
    for e in range(4):
        Wg, Wu, Wd = (oracle.decode_routed(L, n, e) for n in ("gate", "up", "down"))
        G = x @ Wg.T
        ref += p[:, e:e + 1] * ((G * expit(G) * (x @ Wu.T)) @ Wd.T)
    r = oracle.forward(L, x, logits)
    assert np.allclose(np.stack([r["y"][t] for t in range(3)]), ref, rtol=1e-12, atol=1e-14)


def test_zero_routed_blocks_leave_shared_only():
    spec = LayerSpec(256, 128, 4, 2, 64, "q2k")
    L = _tiny_layer(spec)
    for n in ("gate", "up", "down"):
        getattr(L, n).zero_()
    L._host_cache.clear()
    x = make_x(4, 256, seed=10, dtype="fp32").numpy().astype(np.float64)
    logits = make_logits(4, 4, seed=10).numpy()
    r = oracle.forward(L, x, logits)
    Wg, Wu, Wd = (oracle.bf16_bits_to_float64(L.shared(n)) for n in ("sh_gate", "sh_up", "sh_down"))
    G = x @ Wg.T
    ref = (G * expit(G) * (x @ Wu.T)) @ Wd.T
    got = np.stack([r["y"][t] for t in range(4)])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    assert all(np.all(o == 0) for o in r["o"].values())


def test_combine_linear_in_weights():
    rng = np.random.default_rng(14)
    o = rng.standard_normal((4, 32))
    s = rng.standard_normal(32)
    w1 = rng.random(4)
    w2 = rng.random(4)
    a, b = 0.3, 1.7
    lhs = oracle.combine(a * w1 + b * w2, o, None)
    rhs = a * oracle.combine(w1, o, None) + b * oracle.combine(w2, o, None)
    assert np.allclose(lhs, rhs, rtol=1e-13, atol=1e-13)
    assert np.allclose(oracle.combine(w1, o, s) - oracle.combine(w1, o, None), s, atol=1e-14)
    assert np.allclose(oracle.combine(w1, o, None), w1 @ o, rtol=1e-13, atol=1e-14)


def test_evaluation_orders_agree():
    """Per-token (definition) and expert-outer orders on a skewed mid-size layer."""
    spec = LayerSpec(512, 256, 16, 4, 128, "q2k")
    L = _tiny_layer(spec, seed=15)
    x = make_x(24, 512, seed=16, dtype="bf16").float().numpy()
    logits = make_logits(24, 16, seed=17, zipf_s=1.1).numpy()
    r = oracle.forward(L, x, logits)
    Y = oracle.forward_expert_outer(L, x, logits)
    got = np.stack([r["y"][t] for t in range(24)])
    err = np.max(np.abs(got - Y)) / np.max(np.abs(Y))
    assert err < 1e-12, err


def test_mxfp4_layer_orders_agree_and_mx8_close():
    spec = LayerSpec(256, 128, 8, 2, 64, "mxfp4")
    L = _tiny_layer(spec, seed=18)
    x = make_x(8, 256, seed=19, dtype="bf16").float().numpy()
    logits = make_logits(8, 8, seed=20).numpy()
    r = oracle.forward(L, x, logits)
    Y = oracle.forward_expert_outer(L, x, logits)
    got = np.stack([r["y"][t] for t in range(8)])
    assert np.max(np.abs(got - Y)) / np.max(np.abs(Y)) < 1e-12
    # the fp8-operand reading moves the output by a few percent at most
    Y8 = oracle.forward_expert_outer(L, x, logits, mx8=True)
    rel = np.max(np.abs(Y8 - Y), axis=1) / np.max(np.abs(Y), axis=1)
    assert 0 < rel.max() < 0.1


def test_mx8_orders_agree():
    """fp8-operand reading: the per-token order (the definition, quantizing
    each token's x and each pair's h) and the expert-outer order (quantizing
    the batched X and H rows) agree to 1e-12, with a shared expert and
    Zipf-skewed routing."""
    spec = LayerSpec(256, 128, 8, 3, 64, "mxfp4")
    L = _tiny_layer(spec, seed=21)
    x = make_x(20, 256, seed=22, dtype="bf16").float().numpy()
    logits = make_logits(20, 8, seed=23, zipf_s=1.1).numpy()
    r = oracle.forward(L, x, logits, mx8=True)
    Y8 = oracle.forward_expert_outer(L, x, logits, mx8=True)
    got = np.stack([r["y"][t] for t in range(20)])
    assert np.max(np.abs(got - Y8)) / np.max(np.abs(Y8)) < 1e-12
    # and both differ from the bf16-operand layer (the quantization is applied)
    Y = oracle.forward_expert_outer(L, x, logits)
    assert np.max(np.abs(Y8 - Y)) / np.max(np.abs(Y)) > 1e-3


class _GoldenMx8Layer:
    """The hand-worked MXFP8 layer of tests/golden/mx8_layer.json."""

    def __init__(self):
        g = load_golden("mx8_layer.json")
        sp = g["layer"]
        self.spec = LayerSpec(sp["hidden"], sp["ffn"], sp["n_experts"], sp["top_k"], sp["shared_ffn"], sp["wfmt"])
        H, F = sp["hidden"], sp["ffn"]
        gate = np.zeros((F, H // 2), dtype=np.uint8)
        gate[:, 0] = 0x20                         # column 1 = 1.0
        up = np.zeros((F, H // 2), dtype=np.uint8)
        up[:, 1] = 0x04                           # column 2 = 2.0
        down = np.zeros((H, F // 2), dtype=np.uint8)
        for r in range(H):                        # column r = 0.5
            down[r, r // 2] = 0x01 if r % 2 == 0 else 0x10
        sc = lambda rows, K: np.full((rows, K // 32), 127, dtype=np.uint8)
        self._m = {"gate": (gate, sc(F, H)), "up": (up, sc(F, H)), "down": (down, sc(H, F))}
        self.golden = g

    def routed(self, name, e):
        assert e == 0
        return self._m[name]

    def shared(self, name):
        return None


def test_mx8_layer_golden():
    L = _GoldenMx8Layer()
    g = L.golden
    x = np.zeros((1, 32))
    x[0, :3] = g["x"]
    logits = np.array([g["logits"]], dtype=np.float32)
    # the quantized activations
    xv, xe = oracle.mxfp8_quantize(x)
    assert xe.tolist() == [[-7]]
    assert (xv[0, :3] * 2.0 ** -7).tolist() == g["x_quantized"]
    r = oracle.forward(L, x, logits, mx8=True)
    h = r["h"][(0, 0)]
    assert np.allclose(h, g["h_before_quantization"], rtol=1e-15, atol=0)
    hv, he = oracle.mxfp8_quantize(h[None, :])
    assert he.tolist() == [[-10]] and np.all(hv * 2.0 ** -10 == g["h_quantized"])
    assert np.all(r["y"][0] == g["y"])
    assert np.all(oracle.forward_expert_outer(L, x, logits, mx8=True)[0] == g["y"])
    # without the fp8 operands the same layer gives h unquantized: y = h / 2
    r0 = oracle.forward(L, x, logits)
    assert np.all(r0["y"][0] != g["y"])


def test_q4k_layer_identities():
    """Q4K experts: the single-expert layer is the dense SwiGLU FFN of the
    decoded matrices, and per-token, expert-outer and dense-mixture
    evaluations of a routed layer agree."""
    spec1 = LayerSpec(256, 256, 1, 1, 0, "q4k")
    L1 = _tiny_layer(spec1, seed=24)
    x = make_x(5, 256, seed=25, dtype="fp32").numpy().astype(np.float64)
    r = oracle.forward(L1, x, np.zeros((5, 1), dtype=np.float32))
    Wg, Wu, Wd = (oracle.decode_routed(L1, n, 0) for n in ("gate", "up", "down"))
    G = x @ Wg.T
    ref = (G * expit(G) * (x @ Wu.T)) @ Wd.T
    assert np.allclose(np.stack([r["y"][t] for t in range(5)]), ref, rtol=1e-12, atol=1e-14)
    spec = LayerSpec(512, 256, 8, 2, 256, "q4k")
    L = _tiny_layer(spec, seed=26)
    x = make_x(12, 512, seed=27, dtype="bf16").float().numpy()
    logits = make_logits(12, 8, seed=28, zipf_s=1.1).numpy()
    r = oracle.forward(L, x, logits)
    got = np.stack([r["y"][t] for t in range(12)])
    Y = oracle.forward_expert_outer(L, x, logits)
    D = oracle.dense_mixture(L, x, logits)
    assert np.max(np.abs(got - Y)) / np.max(np.abs(Y)) < 1e-12
    assert np.max(np.abs(got - D)) / np.max(np.abs(D)) < 1e-12
