"""GPU parity of the MXFP4 expert path on fp8 operands (scaled matrix
instructions) against the fp64 oracle with MXFP8-quantized x and h.

- ds4moe_quantize_mxfp8: bit-exact with the oracle's quantizer (codes by
  value, scale bytes exactly), including ties, saturation, all-zero blocks and
  blocks below E8M0's range.
- forward with mma_dtype = FP8_E4M3: per-token infinity-norm relative error
  <= 2e-2 against oracle.forward(..., mx8=True) on every token of small layers
  (ragged token tiles, split chunks, several row blocks, one-stage
  reductions); the 4096-token prefill layer is checked in
  test_gpu_fullsize.py.
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


def _quantize(x_bf16):
    n = x_bf16.numel()
    xd = x_bf16.contiguous().to(DEV)
    codes = torch.full((n,), 0x7F, dtype=torch.uint8, device=DEV)
    scales = torch.full((n // 32,), 0xFF, dtype=torch.uint8, device=DEV)
    ds4.quantize_mxfp8(xd, n, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu(), scales.cpu()


def test_quantize_mxfp8_bitexact():
    rng = np.random.default_rng(71)
    blocks = []
    # magnitudes over a wide exponent range, one scale per block
    blocks.append(rng.standard_normal((512, 32)) * np.exp2(rng.integers(-40, 40, size=(512, 1))))
    z = np.zeros((4, 32))
    z[1, 7] = -0.0
    blocks.append(z)                                            # all-zero blocks
    tiny = np.zeros((3, 32))
    tiny[0, :4] = [2.0**-125, -2.0**-130, 2.0**-133, 0.0]      # below E8M0's range: scale held at 2^-127
    tiny[1, :] = 2.0**-126 * rng.standard_normal(32)
    tiny[2, 0] = 3.0e38
    blocks.append(tiny)
    sat = np.zeros((2, 32))
    sat[0, :] = np.linspace(1.0, 1.9921875, 32)                 # amax just below 2: saturates to 448
    sat[1, :] = np.linspace(-4.0, 4.0, 32)                      # amax a power of two
    blocks.append(sat)
    x = torch.from_numpy(np.concatenate(blocks).astype(np.float32)).to(torch.bfloat16).reshape(-1)
    codes, scales = _quantize(x)
    vals, ex = oracle.mxfp8_quantize(x.float().numpy().astype(np.float64).reshape(-1, 32))
    got_vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(-1, 32)
    assert np.array_equal(scales.numpy().astype(np.int64), ex.reshape(-1) + 127)
    assert np.array_equal(got_vals, vals)
    # non-zero codes bit for bit (the oracle's values re-encoded exactly)
    ref_codes = torch.from_numpy(vals.reshape(-1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nz = vals.reshape(-1) != 0
    assert np.array_equal(codes.numpy()[nz], ref_codes[nz])


def test_quantize_mxfp8_sizes():
    """Ragged element counts over the launch's 64-block workgroups, and n = 0."""
    for n in (32, 96, 2048 + 32, 64 * 32 * 3 + 160):
        x = make_x(1, n, seed=n, dtype="bf16").reshape(-1)
        codes, scales = _quantize(x)
        vals, ex = oracle.mxfp8_quantize(x.float().numpy().astype(np.float64).reshape(-1, 32))
        assert np.array_equal(scales.numpy().astype(np.int64), ex.reshape(-1) + 127)
        assert np.array_equal(codes.view(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(-1, 32), vals)
    e = torch.zeros(16, dtype=torch.uint8, device=DEV)
    ds4.quantize_mxfp8(e, 0, e, e)
    with pytest.raises(ds4.Ds4MoeError):
        ds4.quantize_mxfp8(e, 48, e, e)


def _forward(dl, cfg, T, x, logits):
    y = torch.full((T, dl.spec.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds4.forward(cfg, weights(dl), T, x.to(DEV), logits.to(DEV), y, workspace(cfg, T))
    torch.cuda.synchronize()
    return y


def _check(layer, dl, T, algo="grouped", seed=0, zipf=None, tokens=None):
    spec = layer.spec
    x = make_x(T, spec.hidden, seed=500 + seed, dtype="bf16")
    logits = make_logits(T, spec.n_experts, seed=600 + seed, zipf_s=zipf)
    y = _forward(dl, config(spec, algo=algo, mma="fp8"), T, x, logits)
    assert torch.isfinite(y.float()).all()
    r = oracle.forward(layer, x.float().numpy(), logits.numpy(), tokens=tokens, mx8=True)
    toks = sorted(r["y"])
    ref = np.stack([r["y"][t] for t in toks])
    err = rowwise_rel_err(y.float().cpu().numpy()[toks], ref)
    print(f"  T={T} algo={algo} tokens={len(toks)} err={err:.3e}", flush=True)
    return err


SMALL = [
    # name, spec, T
    ("tiny", LayerSpec(256, 128, 8, 2, 128, "mxfp4"), 16),         # one-stage down reduction
    ("ragged", LayerSpec(768, 384, 16, 4, 256, "mxfp4"), 37),
    ("noshared", LayerSpec(512, 256, 8, 3, 0, "mxfp4"), 45),
    ("split", LayerSpec(512, 256, 4, 2, 256, "mxfp4"), 500),       # experts split into 2-3 chunks
    ("wide", LayerSpec(2048, 2048, 8, 2, 2048, "mxfp4"), 96),      # 16 up / 8 down row blocks
    ("one_token", LayerSpec(1024, 512, 16, 4, 512, "mxfp4"), 1),
]


@pytest.mark.parametrize("name,spec,T", SMALL, ids=[s[0] for s in SMALL])
def test_mx8_small(name, spec, T):
    print(f"mx8 small {name} T={T}", flush=True)
    layer = make_layer(spec, seed=700 + len(name), device="cpu")
    assert _check(layer, to_dev(layer), T, algo="auto" if T == 1 else "grouped") <= TOL


def test_mx8_skewed_tile_counts():
    """Zipf-skewed routing: chunks of 1..12 token tiles in one launch."""
    spec = LayerSpec(256, 256, 24, 3, 128, "mxfp4")
    layer = make_layer(spec, seed=78, device="cpu")
    assert _check(layer, to_dev(layer), 700, seed=3, zipf=1.1) <= TOL


def test_mx8_expert_ffn_stage():
    """expert_out rows of the fp8-operand kernels against the oracle (mx8),
    shared_out against the bf16 shared expert, routing from the oracle."""
    spec = LayerSpec(512, 256, 8, 2, 256, "mxfp4")
    T = 150
    layer = make_layer(spec, seed=81, device="cpu")
    dl = to_dev(layer)
    x = make_x(T, spec.hidden, seed=82, dtype="bf16")
    idx, _ = oracle.route(make_logits(T, 8, seed=83).numpy(), 2)
    perm = oracle.permute(idx, 8)
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    cfg = config(spec, algo="grouped", mma="fp8")
    eo = torch.full((T * 2, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    so = torch.full((T, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds4.expert_ffn(cfg, weights(dl), T, x.to(DEV), i32(perm["offsets"]), i32(perm["sorted_pair"]),
                   i32(perm["active"]), eo, so, workspace(cfg, T))
    torch.cuda.synchronize()
    o, _ = oracle.expert_outputs(layer, x.float().numpy(), idx, mx8=True)
    ref_eo = np.stack([o[(int(p) // 2, int(p) % 2)] for p in perm["sorted_pair"]])
    err8 = rowwise_rel_err(eo.float().cpu().numpy(), ref_eo)
    assert err8 <= TOL
    # the result follows the fp8 reading, not the bf16-operand one: the MXFP8
    # rounding of x and h (~3% rms per element) dominates the distance to the
    # unquantized oracle
    ob, _ = oracle.expert_outputs(layer, x.float().numpy(), idx)
    ref_bf = np.stack([ob[(int(p) // 2, int(p) % 2)] for p in perm["sorted_pair"]])
    err_bf = rowwise_rel_err(eo.float().cpu().numpy(), ref_bf)
    print(f"  expert_out err vs mx8 oracle {err8:.3e}, vs unquantized oracle {err_bf:.3e}", flush=True)
    assert err8 < 0.5 * err_bf
    s = oracle.shared_outputs(layer, x.float().numpy())
    assert rowwise_rel_err(so.float().cpu().numpy(), np.stack([s[t] for t in range(T)])) <= TOL


def test_mx8_deterministic():
    spec = LayerSpec(512, 256, 4, 2, 256, "mxfp4")
    T = 300
    dl = to_dev(make_layer(spec, seed=91, device="cpu"))
    x = make_x(T, spec.hidden, seed=92, dtype="bf16")
    logits = make_logits(T, 4, seed=93)
    cfg = config(spec, algo="grouped", mma="fp8")
    y1 = _forward(dl, cfg, T, x, logits)
    y2 = _forward(dl, cfg, T, x, logits)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
