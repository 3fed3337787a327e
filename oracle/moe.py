"""Oracle for one routed-MoE layer: route, permute, expert FFN, shared expert,
combine.  Plain fp64 numpy, one token at a time.

TEST INFRASTRUCTURE: see the package docstring.

A *layer* here is any object with attributes ``spec`` (hidden, ffn, n_experts,
top_k, shared_ffn, wfmt) and the data accessors ``routed(name, e)`` ->
(bytes, scales-or-None) and ``shared(name)`` -> bf16 bit patterns or None.
"""
import numpy as np

from .formats import q2k_decode_matrix, q4k_decode_matrix, mxfp4_decode_matrix, bf16_bits_to_float64, mxfp8_quantize


# ---------------------------------------------------------------- routing ----
def router_logits(x, router_w):
    """Router projection: logits[t][e] = sum_h router_w[e][h] * x[t][h].

    The pages keep the router, like the other projections, at original
    precision while only the routed experts are quantized (hysenlabs
    "DwarfStar実地分析", section "GGUFの対応範囲は意図的に狭い").  Reading:
    the router matrix is stored in bf16, [E][H] (one row per expert), and is
    applied to the token's activations as a plain matrix-vector product.
    Here the product is taken in fp64 on the exact values given (bf16 or fp32
    inputs convert exactly), so the only rounding is fp64's.

    x: [T][H], router_w: [E][H] (values, not bit patterns).  Returns
    float64 [T][E].
    """
    xv = np.asarray(x, dtype=np.float64)
    wv = np.asarray(router_w, dtype=np.float64)
    if xv.ndim != 2 or wv.ndim != 2 or xv.shape[1] != wv.shape[1]:
        raise ValueError("need x [T][H] and router_w [E][H]")
    return xv @ wv.T


def route(logits, k: int):
    """Top-k routing of each token.

    Reading of the router (the pages only say routing stays at original
    precision: hysenlabs "DwarfStar実地分析", section
    "GGUFの対応範囲は意図的に狭い"): softmax over the E logits, keep the k
    largest with ties broken towards the lower expert index, renormalise over
    the kept ones.  Softmax is monotonic, so selection is made on the logits
    themselves: expert i is kept iff fewer than k experts j beat it, where j
    beats i when l_j > l_i, or l_j == l_i and j < i (numeric comparison, so
    -0 == +0).  Slot j of a token holds the expert whose rank is j under that
    order.  Weights: w_j = exp(l_{S_j} - l_{S_0}) / sum_i exp(l_{S_i} - l_{S_0}),
    which equals softmax -> select -> renormalise.

    Returns (idx int64 [T][k], w float64 [T][k]).
    """
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    ar = np.arange(E)
    idx = np.zeros((T, k), dtype=np.int64)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = l[t]
        beats = (row[None, :] > row[:, None]) | ((row[None, :] == row[:, None]) & (ar[None, :] < ar[:, None]))
        rank = beats.sum(axis=1)                       # rank[i] = #experts beating i
        for i in range(E):
            if rank[i] < k:
                idx[t, rank[i]] = i
        sel = row[idx[t]]
        ex = np.exp(sel - sel[0])
        w[t] = ex / ex.sum()
    return idx, w


def route_softmax_chain(logits, k: int):
    """The literal chain: full softmax over E, pick the slots ``route`` picks,
    divide by their sum.  Used to check ``route``'s shortcut."""
    idx, _ = route(logits, k)
    l = np.asarray(logits, dtype=np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx, axis=1)
    return idx, sel / sel.sum(axis=1, keepdims=True)


# ------------------------------------------------------------ permutation ----
def permute(idx, E: int):
    """Expert-major, token-stable order of the T*k (token, slot) pairs.

    Pair id p = t*k + j.  counts[e] = #pairs routed to e; offsets = exclusive
    prefix sum (offsets[E] = T*k); rows of ``sorted_pair`` list, for e
    ascending and then t ascending, the pair of token t routed to e;
    ``pair_pos`` is its inverse; ``active`` = [n, ids of experts with a
    non-zero count, ascending].
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    counts = np.array([(idx == e).sum() for e in range(E)], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_pair = []
    for e in range(E):
        ts, js = np.nonzero(idx == e)                  # row-major: ascending t
        sorted_pair.extend((ts * k + js).tolist())
    sorted_pair = np.array(sorted_pair, dtype=np.int64)
    pair_pos = np.empty(T * k, dtype=np.int64)
    pair_pos[sorted_pair] = np.arange(T * k)
    act = [e for e in range(E) if counts[e] > 0]
    active = np.array([len(act)] + act, dtype=np.int64)
    return dict(counts=counts, offsets=offsets, sorted_pair=sorted_pair, pair_pos=pair_pos,
                active=active)


# -------------------------------------------------------------------- FFN ----
def silu(g):
    """silu(g) = g / (1 + e^-g)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ffn(Wg, Wu, Wd, x):
    """One expert on one token: h = silu(W_g x) * (W_u x), o = W_d h (fp64).
    SwiGLU is this library's reading of the expert activation; the gate is the
    silu branch and there is no clamp."""
    x = np.asarray(x, dtype=np.float64)
    g = Wg @ x
    u = Wu @ x
    h = silu(g) * u
    return Wd @ h, h


def decode_routed(layer, name: str, e: int) -> np.ndarray:
    """Expert e's matrix ``name`` (gate/up: [F][H]; down: [H][F]) decoded
    exactly to float64 from its Q2K, Q4K or MXFP4 bytes."""
    sp = layer.spec
    rows, K = (sp.ffn, sp.hidden) if name in ("gate", "up") else (sp.hidden, sp.ffn)
    data, scales = layer.routed(name, e)
    if sp.wfmt == "q2k":
        return q2k_decode_matrix(data, rows, K)
    if sp.wfmt == "mxfp4":
        return mxfp4_decode_matrix(data, scales, rows, K)
    if sp.wfmt == "q4k":
        return q4k_decode_matrix(data, scales, rows, K)
    raise ValueError(sp.wfmt)


def decode_shared(layer, name: str):
    bits = layer.shared(name)
    return None if bits is None else bf16_bits_to_float64(bits)


def _act(x, mx8: bool):
    """Activation as the expert sees it: as given, or MXFP8-E4M3 quantized
    along K when the fp8-operand path is asked for."""
    x = np.asarray(x, dtype=np.float64)
    if not mx8:
        return x
    vals, exps = mxfp8_quantize(x)
    return vals * np.repeat(np.exp2(exps.astype(np.float64)), 32, axis=-1)


def expert_outputs(layer, x, idx, tokens=None, mx8: bool = False, experts=None):
    """o[(t, j)] = W_d^e h for every requested token t and slot j (e = idx[t][j]).

    Pairs are evaluated one at a time with matrix-vector products; experts are
    decoded once per call and reused across the pairs that need them (that
    changes no arithmetic).  With ``mx8`` the expert's inputs x and h are first
    quantized to MXFP8-E4M3 (the fp8-operand reading of the MXFP4 path).
    ``experts`` (a set of ids), when given, keeps only the pairs routed to
    those experts, so that disjoint sets can be evaluated separately.
    Returns ({(t, j): o float64 [H]}, {(t, j): h float64 [F]}).
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    T, k = idx.shape
    tokens = range(T) if tokens is None else tokens
    need = {}
    for t in tokens:
        for j in range(k):
            e = int(idx[t, j])
            if experts is None or e in experts:
                need.setdefault(e, []).append((t, j))
    out, hs = {}, {}
    for e in sorted(need):
        Wg = decode_routed(layer, "gate", e)
        Wu = decode_routed(layer, "up", e)
        Wd = decode_routed(layer, "down", e)
        for (t, j) in need[e]:
            xt = _act(x[t], mx8)
            g = Wg @ xt
            u = Wu @ xt
            h = silu(g) * u
            hs[(t, j)] = h
            out[(t, j)] = Wd @ _act(h, mx8)
        del Wg, Wu, Wd
    return out, hs


def shared_outputs(layer, x, tokens=None):
    """Shared expert, always on, bf16 weights decoded exactly:
    s_t = W_d^s (silu(W_g^s x_t) * W_u^s x_t).  Returns {t: s float64 [H]} or
    None when the layer has no shared expert."""
    if not layer.spec.shared_ffn:
        return None
    x = np.asarray(x, dtype=np.float64)
    Wg, Wu, Wd = (decode_shared(layer, n) for n in ("sh_gate", "sh_up", "sh_down"))
    tokens = range(x.shape[0]) if tokens is None else tokens
    return {t: swiglu_ffn(Wg, Wu, Wd, x[t])[0] for t in tokens}


def combine(w, o, s=None):
    """y_t = s_t + sum_j w_{t,j} o_{t,j} (fp64), for one token: w [k], o [k][H],
    s [H] or None.  The shared expert is added with weight 1."""
    w = np.asarray(w, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    y = np.zeros(o.shape[1], dtype=np.float64) if s is None else np.array(s, dtype=np.float64)
    for j in range(w.shape[0]):
        y = y + w[j] * o[j]
    return y


def forward(layer, x, logits, tokens=None, mx8: bool = False):
    """Whole layer for the requested tokens (all by default), per-token order.

    Returns dict(idx, w, perm, y {t: [H]}, o {(t,j): [H]}, h {(t,j): [F]},
    s {t: [H]} or None)."""
    sp = layer.spec
    idx, w = route(logits, sp.top_k)
    perm = permute(idx, sp.n_experts)
    T = idx.shape[0]
    tokens = list(range(T)) if tokens is None else list(tokens)
    o, h = expert_outputs(layer, x, idx, tokens, mx8=mx8)
    s = shared_outputs(layer, x, tokens)
    y = {}
    for t in tokens:
        y[t] = combine(w[t], np.stack([o[(t, j)] for j in range(sp.top_k)]),
                       None if s is None else s[t])
    return dict(idx=idx, w=w, perm=perm, y=y, o=o, h=h, s=s)


def forward_expert_outer(layer, x, logits, mx8: bool = False, experts=None, shared: bool = True, routing=None):
    """Same layer, expert-outer order: each expert is decoded once and its
    tokens go through it together as fp64 matrix products (identical math up
    to summation order inside the products).  Returns y float64 [T][H].

    ``experts`` (a set of ids) and ``shared=False`` restrict the sum to those
    experts' terms and leave out the shared expert: a partial sum, used to
    time a bounded sample of the work.  ``routing`` = (idx, w) from ``route``
    on the same logits skips routing them again."""
    sp = layer.spec
    x = np.asarray(x, dtype=np.float64)
    idx, w = route(logits, sp.top_k) if routing is None else routing
    T = x.shape[0]
    y = np.zeros((T, sp.hidden), dtype=np.float64)
    for e in range(sp.n_experts):
        if experts is not None and e not in experts:
            continue
        ts, js = np.nonzero(idx == e)
        if ts.size == 0:
            continue
        Wg = decode_routed(layer, "gate", e)
        Wu = decode_routed(layer, "up", e)
        Wd = decode_routed(layer, "down", e)
        X = _act(x[ts], mx8)
        H = silu(X @ Wg.T) * (X @ Wu.T)
        O = _act(H, mx8) @ Wd.T
        y[ts] += w[ts, js][:, None] * O
    if sp.shared_ffn and shared:
        Wg, Wu, Wd = (decode_shared(layer, n) for n in ("sh_gate", "sh_up", "sh_down"))
        y += (silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    return y


def dense_mixture(layer, x, logits):
    """Y_t = sum_e M[t,e] FFN_e(x_t) over *all* E experts, with M the routing
    weights scattered to a dense [T][E] matrix (zero for unselected experts),
    plus the shared expert.  A second route to the same layer output, used to
    pin ``forward``."""
    sp = layer.spec
    x = np.asarray(x, dtype=np.float64)
    idx, w = route(logits, sp.top_k)
    T = x.shape[0]
    M = np.zeros((T, sp.n_experts))
    np.put_along_axis(M, idx, w, axis=1)
    outs = []
    for e in range(sp.n_experts):
        Wg = decode_routed(layer, "gate", e)
        Wu = decode_routed(layer, "up", e)
        Wd = decode_routed(layer, "down", e)
        outs.append((silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T)      # [T][H]
    F = np.stack(outs)                                          # [E][T][H]
    Y = np.einsum("te,eth->th", M, F)
    if sp.shared_ffn:
        Wg, Wu, Wd = (decode_shared(layer, n) for n in ("sh_gate", "sh_up", "sh_down"))
        Y = Y + (silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    return Y
