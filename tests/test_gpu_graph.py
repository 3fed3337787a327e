"""ds4moe_forward under HIP graph capture.

The forward launches only kernels on the caller's stream: no memset, no
allocation, no host synchronization; the grouped GEMM's work counters are
cleared by its plan kernel.  A captured forward is replayed several times,
with fresh router logits copied into the captured buffer, eager library work
and synchronizations between the replays, and every replay must reproduce the
eager output bit for bit.
"""
import pytest
import torch

from synth import LayerSpec, make_layer, make_x, make_logits

pytestmark = pytest.mark.gpu

ds4 = pytest.importorskip("bit_routed_moe_amd")
from helpers import DEV, config, weights, to_dev, workspace  # noqa: E402

CASES = [
    # name, spec, T, mma: the batch-1 path, the GEMV kernels, the grouped
    # GEMM's small-batch layout, its prefill layout (split experts), and MXFP4
    # experts on fp8 operands (the MXFP8 quantizer launch first)
    ("batch1", LayerSpec(1024, 1024, 16, 4, 256, "q2k"), 1, "bf16"),
    ("gemv", LayerSpec(512, 256, 16, 4, 256, "q2k"), 4, "bf16"),
    ("grouped_small", LayerSpec(512, 256, 16, 4, 256, "mxfp4"), 24, "bf16"),
    ("grouped_prefill", LayerSpec(512, 256, 4, 2, 256, "q2k"), 500, "bf16"),
    ("grouped_fp8", LayerSpec(512, 256, 4, 2, 256, "mxfp4"), 300, "fp8"),
]


@pytest.mark.parametrize("name,spec,T,mma", CASES, ids=[c[0] for c in CASES])
def test_forward_graph_replays_match_eager(name, spec, T, mma):
    print(f"graph {name} T={T}", flush=True)
    dl = to_dev(make_layer(spec, seed=400 + T, device="cpu"))
    cfg = config(spec, algo="auto", mma=mma)
    w = weights(dl)
    x = make_x(T, spec.hidden, seed=401, dtype="bf16").to(DEV)
    draws = [make_logits(T, spec.n_experts, seed=402, index=i).to(DEV) for i in range(3)]

    # eager references, one per router draw
    ws_eager = workspace(cfg, T)
    refs = []
    for lg in draws:
        y = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)
        ds4.forward(cfg, w, T, x, lg, y, ws_eager)
        refs.append(y)
    torch.cuda.synchronize()

    # capture on a side stream (default priority), after a warm-up there
    logits = draws[0].clone()
    y = torch.full((T, spec.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = workspace(cfg, T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ds4.forward(cfg, w, T, x, logits, y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds4.forward(cfg, w, T, x, logits, y, ws)
    torch.cuda.synchronize()

    y_other = torch.empty_like(y)
    for rep in range(6):
        i = rep % 3
        logits.copy_(draws[i])
        y.fill_(float("nan"))
        # eager library work on another workspace between the replays
        ds4.forward(cfg, w, T, x, draws[(i + 1) % 3], y_other, ws_eager)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), refs[i].view(torch.int16)), (name, rep)
        assert torch.equal(y_other.view(torch.int16), refs[(i + 1) % 3].view(torch.int16)), (name, rep)


@pytest.mark.parametrize("T", [1, 40], ids=["batch1", "mfma_router"])
def test_router_and_forward_graph_replays_match_eager(T):
    """The router projection and the layer captured together: x -> logits ->
    y, replayed with fresh activations copied into the captured buffer."""
    from synth import make_router_w
    print(f"graph router+forward T={T}", flush=True)
    spec = LayerSpec(1024, 1024, 16, 4, 256, "q2k")
    dl = to_dev(make_layer(spec, seed=450 + T, device="cpu"))
    cfg = config(spec, algo="auto")
    w = weights(dl)
    wr = make_router_w(spec.n_experts, spec.hidden, seed=451).to(DEV)
    xs = [make_x(T, spec.hidden, seed=452, copy=i, dtype="bf16").to(DEV) for i in range(3)]

    def run(x, logits, y, ws):
        ds4.router_logits(cfg, T, x, wr, logits)
        ds4.forward(cfg, w, T, x, logits, y, ws)

    ws_eager = workspace(cfg, T)
    lg_eager = torch.empty((T, spec.n_experts), dtype=torch.float32, device=DEV)
    refs = []
    for x in xs:
        y = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)
        run(x, lg_eager, y, ws_eager)
        refs.append(y)
    torch.cuda.synchronize()

    x = xs[0].clone()
    lg = torch.empty_like(lg_eager)
    y = torch.empty((T, spec.hidden), dtype=torch.bfloat16, device=DEV)
    ws = workspace(cfg, T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(x, lg, y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(x, lg, y, ws)
    torch.cuda.synchronize()

    y_other = torch.empty_like(y)
    for rep in range(6):
        i = rep % 3
        x.copy_(xs[i])
        y.fill_(float("nan"))
        run(xs[(i + 1) % 3], lg_eager, y_other, ws_eager)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), refs[i].view(torch.int16)), (T, rep)
        assert torch.equal(y_other.view(torch.int16), refs[(i + 1) % 3].view(torch.int16)), (T, rep)
