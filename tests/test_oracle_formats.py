"""Pins for the oracle's format decoders (CPU only).

Each check ties the oracle to something other than itself: hand-worked blocks
(tests/golden), an independent library decoder (numpy's binary16, torch's
bf16 and fp8 casts), exhaustive enumeration, and structural invariants.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden, golden_q2k_block
from synth import q2k_encode, mxfp4_encode, q4k_encode


def _bits32(x):
    return int(np.asarray([x], dtype=np.float32).view(np.uint32)[0])


# ---------------------------------------------------------------- fp16 -------
def test_fp16_golden():
    for bits, val in load_golden("fp16_values.json")["cases"]:
        got = float(oracle.fp16_to_float64(int(bits, 16)))
        assert got == val and np.signbit(got) == np.signbit(val), bits


def test_fp16_exhaustive_vs_numpy():
    """All 65536 patterns against numpy's own binary16 decoder."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.fp16_to_float64(bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


# ------------------------------------------------------------ Q2K blocks -----
GOLD = load_golden("q2k_blocks.json")["blocks"]


def _block(bid):
    spec = next(b for b in GOLD if b["id"] == bid)
    return spec, np.frombuffer(golden_q2k_block(spec), dtype=np.uint8)


def test_q2k_block_sizes():
    for spec in GOLD:
        assert len(golden_q2k_block(spec)) == 84


def test_q2k_B1_pattern():
    spec, b = _block("B1")
    w = oracle.q2k_decode(b)
    assert w.shape == (256,)
    assert np.array_equal(w, np.tile(spec["pattern"], 64))
    assert w.sum() == spec["sum"]


def test_q2k_B2_groups():
    spec, b = _block("B2")
    w = oracle.q2k_decode(b).reshape(16, 16)
    assert np.array_equal(w, np.repeat(np.array(spec["group_values"])[:, None], 16, axis=1))


@pytest.mark.parametrize("bid", ["B3", "B5", "B6"])
def test_q2k_rounding_cases(bid):
    spec, b = _block(bid)
    w = oracle.q2k_decode(b)
    e = spec["element"]
    assert w[e] == spec["exact"]
    w32 = oracle.fp32_round(w[e])
    assert _bits32(w32) == int(spec["w32_bits"], 16)
    if "bf16_bits" in spec:
        assert int(oracle.bf16_bits_from_fp32(w32)) == int(spec["bf16_bits"], 16)
    if "bf16_of_exact_bits" in spec:
        # Rounding the exact value straight to bf16 is a different (rejected)
        # reading: the exact value lies above the midpoint of its bf16
        # neighbours, so it would round up to the other pattern.
        lo = float(oracle.bf16_bits_to_float64(int(spec["bf16_bits"], 16)))
        hi = float(oracle.bf16_bits_to_float64(int(spec["bf16_of_exact_bits"], 16)))
        assert lo < (lo + hi) / 2 < w[e] < hi and w32 == (lo + hi) / 2
    if "rest" in spec:
        assert np.all(w[16:] == spec["rest"])


def test_q2k_B4_negative_d_and_signed_zero():
    spec, b = _block("B4")
    w32 = oracle.fp32_round(oracle.q2k_decode(b)[:2])
    assert [hex(_bits32(v)) for v in w32] == spec["w32_bits_first2"]


def test_q2k_B7_zero_block():
    _, b = _block("B7")
    w = oracle.q2k_decode(b)
    assert np.all(w == 0) and not np.any(np.signbit(w))


def test_q2k_group_invariant_random_bytes():
    """Any block: within a group at most 4 distinct values, spaced by d*s."""
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 256, size=(64, 84), dtype=np.uint8)
    raw[:, 81] &= 0x3B           # keep d, dmin finite (exponent < 31)
    raw[:, 83] &= 0x3B
    w = oracle.q2k_decode(raw.reshape(-1)).reshape(64, 16, 16)
    for bi in range(64):
        d = oracle.fp16_to_float64(int(raw[bi, 80]) | int(raw[bi, 81]) << 8)
        for g in range(16):
            s = raw[bi, g] & 0xF
            vals = np.unique(w[bi, g])
            assert len(vals) <= 4
            if len(vals) > 1:
                steps = np.diff(vals) / (d * s)
                assert np.allclose(steps, np.round(steps)) and np.all(np.round(steps) >= 1)


def test_q2k_matrix_flat_mapping():
    """Rows shorter than a super-block (K = 128): weight (r, c) is flat element r*K + c."""
    rng = np.random.default_rng(2)
    w = torch.from_numpy(rng.standard_normal((4, 128)).astype(np.float32))
    data = q2k_encode(w).numpy().reshape(-1)
    flat = oracle.q2k_decode(data)
    mat = oracle.q2k_decode_matrix(data, 4, 128)
    assert np.array_equal(mat.reshape(-1), flat)
    assert np.array_equal(mat[1], flat[128:256])


def test_q2k_encode_decode_roundtrip_quality():
    """The fixture encoder and the oracle decoder were written apart; a field
    swapped in either would wreck the reconstruction.  2-bit min/max groups on
    Gaussian weights keep the error well under the weights' spread."""
    rng = np.random.default_rng(3)
    w = rng.standard_normal((64, 256)).astype(np.float32) * 0.02
    data = q2k_encode(torch.from_numpy(w)).numpy().reshape(-1)
    wh = oracle.q2k_decode(data).reshape(64, 256)
    rel = np.sqrt(np.mean((wh - w) ** 2)) / np.std(w)
    assert 0.15 < rel < 0.45, rel
    # per-group: every weight lies within one step (d*s) of its reconstruction
    assert np.corrcoef(wh.ravel(), w.ravel())[0, 1] > 0.9


# ------------------------------------------------------------ Q4K blocks -----
GOLD4 = load_golden("q4k_blocks.json")["blocks"]


def _expand(lst, n):
    out, i = [], 0
    while i < len(lst):
        v = int(lst[i], 16)
        if i + 1 < len(lst) and isinstance(lst[i + 1], int):
            out += [v] * lst[i + 1]
            i += 2
        else:
            out.append(v)
            i += 1
    assert len(out) == n
    return out


def _q4_block(bid):
    """(spec, codes uint8 [128], params uint8 [20]) of a golden Q4K block."""
    spec = next(b for b in GOLD4 if b["id"] == bid)
    if spec.get("codes") == "staircase":
        codes = [(2 * j) % 16 | (((2 * j + 1) % 16) << 4) for j in range(128)]
    else:
        head = [int(h, 16) for h in spec["codes_head"]]
        codes = head + [int(spec["codes_fill"], 16)] * (128 - len(head))
    d, dm = int(spec["d"], 16), int(spec["dmin"], 16)
    params = _expand(spec["scales"], 16) + [d & 0xFF, d >> 8, dm & 0xFF, dm >> 8]
    return spec, np.array(codes, dtype=np.uint8), np.array(params, dtype=np.uint8)


def _q4_decode(codes, params):
    return oracle.q4k_decode_matrix(codes, params, 1, 256)[0]


def test_q4k_K1_staircase_and_nibble_order():
    spec, c, p = _q4_block("K1")
    w = _q4_decode(c, p)
    assert np.array_equal(w, np.tile(spec["pattern"], 16))
    assert w.sum() == spec["sum"]


def test_q4k_K2_groups():
    spec, c, p = _q4_block("K2")
    w = _q4_decode(c, p).reshape(16, 16)
    assert np.array_equal(w, np.repeat(np.array(spec["group_values"])[:, None], 16, axis=1))


@pytest.mark.parametrize("bid", ["K3", "K5", "K6"])
def test_q4k_rounding_cases(bid):
    spec, c, p = _q4_block(bid)
    w = _q4_decode(c, p)
    e = spec["element"]
    assert w[e] == spec["exact"]
    w32 = oracle.fp32_round(w[e])
    assert _bits32(w32) == int(spec["w32_bits"], 16)
    if "bf16_bits" in spec:
        assert int(oracle.bf16_bits_from_fp32(w32)) == int(spec["bf16_bits"], 16)
    if "bf16_of_exact_bits" in spec:
        lo = float(oracle.bf16_bits_to_float64(int(spec["bf16_bits"], 16)))
        hi = float(oracle.bf16_bits_to_float64(int(spec["bf16_of_exact_bits"], 16)))
        assert lo < (lo + hi) / 2 < w[e] < hi and w32 == (lo + hi) / 2
    if "rest" in spec:
        assert np.all(w[16:] == spec["rest"])


def test_q4k_K4_negative_d_and_signed_zero():
    spec, c, p = _q4_block("K4")
    w32 = oracle.fp32_round(_q4_decode(c, p)[:2])
    assert [hex(_bits32(v)) for v in w32] == spec["w32_bits_first2"]


def test_q4k_K7_zero_block():
    _, c, p = _q4_block("K7")
    w = _q4_decode(c, p)
    assert np.all(w == 0) and not np.any(np.signbit(w))


def test_q4k_super_block_indexing():
    """A [2][512] matrix: element (r, c) takes its parameters from record
    c // 256 of row r and its code from byte r*256 + c//2."""
    _, c1, p1 = _q4_block("K1")
    codes = np.tile(c1, 4)                          # 2 rows x 2 super-blocks of the staircase
    recs = []
    for r in range(2):
        for b in range(2):
            p = p1.copy()
            d = [0x3c00, 0x4000, 0x4200, 0x4400][2 * r + b]   # 1, 2, 3, 4
            p[16], p[17] = d & 0xFF, d >> 8
            recs.append(p)
    W = oracle.q4k_decode_matrix(codes, np.concatenate(recs), 2, 512)
    stair = np.tile(np.arange(16.0), 16)
    for r in range(2):
        for b in range(2):
            assert np.array_equal(W[r, 256 * b:256 * (b + 1)], (2 * r + b + 1) * stair)


def test_q4k_group_invariant_random_bytes():
    """Any block: within a group at most 16 distinct values, spaced by whole
    multiples of d*s."""
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, size=(32, 128), dtype=np.uint8)
    params = rng.integers(0, 256, size=(32, 20), dtype=np.uint8)
    params[:, 17] &= 0x3B
    params[:, 19] &= 0x3B
    W = oracle.q4k_decode_matrix(codes, params, 32, 256).reshape(32, 16, 16)
    for r in range(32):
        d = oracle.fp16_to_float64(int(params[r, 16]) | int(params[r, 17]) << 8)
        for g in range(16):
            s = params[r, g] & 0xF
            vals = np.unique(W[r, g])
            assert len(vals) <= 16
            if len(vals) > 1:
                steps = np.diff(vals) / (d * s)
                assert np.allclose(steps, np.round(steps)) and np.all(np.round(steps) >= 1)


def test_q4k_encode_decode_roundtrip_quality():
    """Encoder and decoder written apart: 4-bit min/max groups on Gaussian
    weights reconstruct to a few percent of the spread (a swapped field would
    wreck it), and better than the 2-bit blocks."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal((64, 512)).astype(np.float32) * 0.02
    c, p = q4k_encode(torch.from_numpy(w))
    wh = oracle.q4k_decode_matrix(c.numpy(), p.numpy(), 64, 512)
    rel = np.sqrt(np.mean((wh - w) ** 2)) / np.std(w)
    assert 0.03 < rel < 0.12, rel
    q2 = oracle.q2k_decode(q2k_encode(torch.from_numpy(w)).numpy().reshape(-1)).reshape(64, 512)
    assert rel < 0.5 * np.sqrt(np.mean((q2 - w) ** 2)) / np.std(w)


# ----------------------------------------------------------------- MXFP4 -----
MX = load_golden("mxfp4_values.json")


def test_e2m1_table():
    got = oracle.e2m1_to_float64(np.arange(16))
    ref = np.array(MX["e2m1_table"])
    assert np.array_equal(got, ref) and np.array_equal(np.signbit(got), np.signbit(ref))


def test_e2m1_vs_torch_fp4():
    """torch's own float4_e2m1fn_x2 decoder, where available."""
    if not hasattr(torch, "float4_e2m1fn_x2"):
        pytest.skip("torch has no float4 dtype")
    packed = torch.tensor([(2 * i + 1) << 4 | (2 * i) for i in range(8)], dtype=torch.uint8)
    try:
        ref = packed.view(torch.float4_e2m1fn_x2).to(torch.float32)
    except (RuntimeError, TypeError, NotImplementedError):
        pytest.skip("torch cannot convert float4 on this build")
    assert np.array_equal(ref.numpy().ravel().astype(np.float64), oracle.e2m1_to_float64(np.arange(16)))


@pytest.mark.parametrize("case", MX["cases"], ids=[c["id"] for c in MX["cases"]])
def test_mxfp4_cases(case):
    codes = np.array([[int(case["code_byte"], 16)] * 16], dtype=np.uint8)
    scales = np.array([[int(case["scale"], 16)]], dtype=np.uint8)
    w = oracle.mxfp4_decode_matrix(codes, scales, 1, 32)[0]
    exp = [float(v) for v in case["values"]]
    for c in range(2):
        if np.isnan(exp[c]):
            assert np.isnan(w[c])
        else:
            assert w[c] == exp[c]
    if "w32_bits" in case:
        assert [_bits32(v) for v in oracle.fp32_round(w[:2])] == [int(h, 16) for h in case["w32_bits"]]


def test_mxfp4_layout_low_nibble_even():
    codes = np.zeros((2, 32), dtype=np.uint8)
    codes[1, 3] = 0x5A                      # row 1, elements 6 (low: 0xA=-1.0) and 7 (high: 5=3.0)
    scales = np.full((2, 2), 127, dtype=np.uint8)
    scales[1, 0] = 128                      # block 0 of row 1 scaled by 2
    w = oracle.mxfp4_decode_matrix(codes, scales, 2, 64)
    assert w[1, 6] == -2.0 and w[1, 7] == 6.0
    assert np.count_nonzero(w) == 2


def test_mxfp4_encode_decode_roundtrip_quality():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((32, 256)).astype(np.float32) * 0.02
    c, s = mxfp4_encode(torch.from_numpy(w))
    wh = oracle.mxfp4_decode_matrix(c.numpy(), s.numpy(), 32, 256)
    rel = np.sqrt(np.mean((wh - w) ** 2)) / np.std(w)
    assert rel < 0.15, rel


# --------------------------------------------------------- rounding ----------
def test_bf16_rounding_vs_torch():
    """RNE on the fp32 bits, against torch's own fp32 -> bf16 cast."""
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
                        np.array([1.00390625, 1.0078125 - 2**-24, 3.0e38, -0.0, 0.0], dtype=np.float32)])
    # exact ties: low 16 bits = 0x8000
    u = rng.integers(0, 2**31, size=4000, dtype=np.uint32)
    u = (u & 0x7F7F0000) | 0x8000
    x = np.concatenate([x, u.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits_from_fp32(x)
    assert np.array_equal(got, ref)


def test_e4m3_vs_torch():
    """OCP E4M3 nearest-even rounding against torch's float8_e4m3fn cast
    within the finite range (torch does not saturate beyond it)."""
    rng = np.random.default_rng(6)
    v = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(2000) * 1e-2,
                        np.array([448.0, -448.0, 2**-9, 2**-10, 3 * 2**-10, 1.0625, 1.1875, 0.0])])
    v = v.astype(np.float32).astype(np.float64)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_round(v)
    assert np.array_equal(got, ref)
    assert np.all(oracle.e4m3_round(np.array([449.0, 464.0, 1e6, -600.0])) == [448, 448, 448, -448])


def test_mxfp8_scale_rule():
    x = np.zeros((2, 64))
    x[0, :32] = np.linspace(-3.0, 3.0, 32)      # amax 3 -> floor(log2 3) = 1 -> X = 2^-7
    x[1, 32:] = 0.0
    vals, ex = oracle.mxfp8_quantize(x)
    assert ex[0, 0] == 1 - 8 and ex[1, 1] == 0 and ex[0, 1] == 0
    assert np.all(vals[1] == 0)
    # element = x / X rounded to E4M3; |x|/X <= 3*128 = 384 stays unsaturated
    assert np.array_equal(vals[0, :32], oracle.e4m3_round(x[0, :32] * 128))


def test_mxfp8_scale_edges():
    """Scale exponent at exact powers of two, just below them (the largest
    element then saturates to 448), and below E8M0's range (held at -127)."""
    x = np.zeros((4, 32))
    x[0, 0] = 4.0                      # amax = 2^2 exactly: X = 2^-6, element 256
    x[1, 0] = 2.0 - 2.0**-7            # floor(log2) = 0: X = 2^-8, 510 -> rounds to 512 -> 448
    x[1, 1] = 1.0                      # 256 exactly
    x[2, 0] = 2.0**-125                # X would be 2^-133: held at 2^-127, element 4
    x[2, 1] = -2.0**-126
    x[3, :] = -0.0                     # signed zeros: an all-zero block
    vals, ex = oracle.mxfp8_quantize(x)
    assert list(ex[:, 0]) == [-6, -8, -127, 0]
    assert vals[0, 0] == 256 and vals[1, 0] == 448 and vals[1, 1] == 256
    assert vals[2, 0] == 4 and vals[2, 1] == -2
    assert np.all(vals[3] == 0)


def test_mxfp8_brute_force_nearest():
    """Every element against a brute-force nearest search over the 253 finite
    E4M3 magnitudes (ties to the even code), on random blocks with a spread of
    magnitudes."""
    mags = []
    for code in range(0x7F):           # 0x7F is NaN in OCP E4M3
        e, mnt = code >> 3, code & 7
        mags.append(mnt * 2.0**-9 if e == 0 else (1 + mnt / 8) * 2.0**(e - 7))
    mags = np.array(mags)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((40, 64)) * np.exp2(rng.integers(-20, 20, size=(40, 1)))
    x[3, 5:9] = 0.0
    vals, ex = oracle.mxfp8_quantize(x)
    X = np.repeat(np.exp2(ex.astype(np.float64)), 32, axis=-1)
    for v, q, s in zip(x.ravel(), vals.ravel(), X.ravel()):
        a = min(abs(v) / s, 448.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert q == np.copysign(mags[code], v) or (q == 0 and mags[code] == 0)
