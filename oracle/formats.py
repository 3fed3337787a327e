"""Oracle decoders for the weight formats, written from their definitions (fp64).

TEST INFRASTRUCTURE: see the package docstring.

Sources.  The pages name the formats only: Q2_K super-blocks for the 2-bit
routed experts, and MXFP4 routed experts kept as DeepSeek published them
(hysenlabs "DwarfStar実地分析", section "GGUFの対応範囲は意図的に狭い";
README mirror "DS4 分布式Shell客户端", section "模型下载").  The Q2K-style block
decoded here is the one this library defines: 256 weights in 16 groups of 16
two-bit codes, a 4-bit scale s and 4-bit min m per group, fp16 d and dmin, and
weight = d*s*q - dmin*m; 84 bytes.  MXFP4 follows the public OCP Microscaling
v1.0 definition (E2M1 elements, one E8M0 scale per 32).
"""
import numpy as np


def fp16_to_float64(bits) -> np.ndarray:
    """IEEE 754 binary16 bit patterns -> float64, from the definition:
    (-1)^s * 2^(e-15) * (1 + f/1024) for 0 < e < 31, (-1)^s * 2^-14 * f/1024 for
    e == 0, infinities and NaN for e == 31."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = (f / 1024.0) * 2.0 ** -14
    special = np.where(f == 0, np.inf, np.nan)
    val = np.where(e == 0, sub, np.where(e == 31, special, normal))
    return sign * val


def q2k_decode(data: np.ndarray, n: int = None) -> np.ndarray:
    """Decode Q2K-style super-blocks (flat uint8, 84 bytes each) to float64.

    Block layout: bytes 0..15 hold group j's scale s_j (low nibble) and min
    m_j (high nibble); bytes 16..79 hold code i (i = 0..255) at byte 16 + i//4,
    bits 2*(i%4); bytes 80..81 and 82..83 are d and dmin as little-endian fp16.
    Weight i = d * s_{i//16} * q_i - dmin * m_{i//16}.
    """
    b = np.asarray(data, dtype=np.uint8).reshape(-1, 84)
    nb = b.shape[0]
    s = (b[:, 0:16] & 0xF).astype(np.float64)          # [nb][16] scale of group j
    m = (b[:, 0:16] >> 4).astype(np.float64)           # [nb][16] min of group j
    codes = b[:, 16:80]                                 # code i: byte i//4, bits 2*(i%4)
    q = np.stack([(codes >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(nb, 16, 16)
    d = fp16_to_float64(b[:, 80].astype(np.int64) | (b[:, 81].astype(np.int64) << 8))
    dmin = fp16_to_float64(b[:, 82].astype(np.int64) | (b[:, 83].astype(np.int64) << 8))
    # d*s and dmin*m are exact in fp64, so (d*s)*q - dmin*m is the closed form
    w = (d[:, None] * s)[:, :, None] * q - (dmin[:, None] * m)[:, :, None]
    w = w.reshape(-1)
    return w if n is None else w[:n]


def q2k_decode_matrix(data: np.ndarray, rows: int, K: int) -> np.ndarray:
    """A [rows][K] matrix stored flat row-major in 256-weight blocks: weight
    (r, c) is element (r*K + c) % 256 of block (r*K + c) // 256."""
    return q2k_decode(data, rows * K).reshape(rows, K)


def q4k_decode_matrix(codes: np.ndarray, params: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Decode a Q4K-style [rows][K] matrix (K % 256 == 0) to float64.

    The pages mention 4-bit expert files beside the 2-bit ones (a stack whose
    last six layers' experts are q4, and a q4 model; README mirror
    "DS4 分布式Shell客户端", section "模型下载") but give no layout.  This
    library's reading is the 2-bit super-block's 4-bit analogue: per 256
    consecutive weights of a row, 16 groups of 16 four-bit codes q (0..15),
    a 4-bit scale s_j and 4-bit min m_j per group, fp16 d and dmin, and
    weight = d * s_j * q - dmin * m_j (148 bytes per 256 weights).  It is
    stored in two arrays, like MXFP4:
      codes  [rows][K/2]: element c of a row in byte c//2, low nibble when c
             is even;
      params [rows][K/256][20]: bytes 0..15 hold group j's s_j (low nibble)
             and m_j (high nibble), bytes 16..17 d and 18..19 dmin as
             little-endian fp16.
    """
    if K % 256:
        raise ValueError("Q4K rows must be whole 256-weight super-blocks")
    c = np.asarray(codes, dtype=np.uint8).reshape(rows, K // 2).astype(np.int64)
    q = np.empty((rows, K), dtype=np.float64)
    q[:, 0::2] = c & 0xF
    q[:, 1::2] = c >> 4
    p = np.asarray(params, dtype=np.uint8).reshape(rows, K // 256, 20).astype(np.int64)
    s = (p[:, :, 0:16] & 0xF).astype(np.float64)        # [rows][K/256][16]
    m = (p[:, :, 0:16] >> 4).astype(np.float64)
    d = fp16_to_float64(p[:, :, 16] | (p[:, :, 17] << 8))        # [rows][K/256]
    dmin = fp16_to_float64(p[:, :, 18] | (p[:, :, 19] << 8))
    # d*s and dmin*m are exact in fp64, so (d*s)*q - dmin*m is the closed form
    a = np.repeat((d[:, :, None] * s).reshape(rows, K // 16), 16, axis=1)
    b = np.repeat((dmin[:, :, None] * m).reshape(rows, K // 16), 16, axis=1)
    return a * q - b


def e2m1_to_float64(nib) -> np.ndarray:
    """OCP E2M1 nibble -> value: sign bit 3, exponent bits 2..1, mantissa bit 0;
    |v| = 0.5*m for exponent 0, else (1 + m/2) * 2^(exponent-1)."""
    n = np.asarray(nib, dtype=np.int64)
    sign = (n >> 3) & 1
    e = (n >> 1) & 3
    mm = (n & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * mm, (1.0 + mm / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return np.where(sign == 1, -mag, mag)


def mxfp4_decode_matrix(codes: np.ndarray, scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    """MXFP4 [rows][K]: codes [rows][K/2] (element c in byte c//2, low nibble
    when c is even), E8M0 scales [rows][K/32] (2^(s-127); 255 is NaN).
    Weight = E2M1(code) * scale of its 32-element block (exact in fp64)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(rows, K // 2).astype(np.int64)
    nib = np.empty((rows, K), dtype=np.int64)
    nib[:, 0::2] = c & 0xF
    nib[:, 1::2] = c >> 4
    v = e2m1_to_float64(nib)
    s = np.asarray(scales, dtype=np.uint8).reshape(rows, K // 32).astype(np.int64)
    X = np.where(s == 255, np.nan, np.exp2(s.astype(np.float64) - 127.0))
    return v * np.repeat(X, 32, axis=1)


def bf16_bits_to_float64(bits) -> np.ndarray:
    """bf16 bit patterns (the top half of an fp32) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp32_round(x) -> np.ndarray:
    """Round float64 to the nearest fp32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits_from_fp32(x32) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even on the fp32 bits (NaN
    inputs keep a quiet NaN pattern)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def e4m3_round(v) -> np.ndarray:
    """Round float64 values to OCP FP8 E4M3 (bias 7, max normal 448, smallest
    subnormal 2^-9), nearest with ties to even, saturating at +-448.  Returns
    the represented values as float64."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # exact exponent: fix floating log2 misses near powers of two
    ex = np.where(np.exp2(ex) > a, ex - 1, ex)
    ex = np.where(np.exp2(ex + 1) <= a, ex + 1, ex)
    ex = np.maximum(ex, -6.0)                 # subnormal range shares 2^-6's spacing
    ulp = np.exp2(ex - 3.0)
    q = np.round(a / ulp) * ulp               # numpy round: half to even
    q = np.minimum(q, 448.0)
    return np.where(v < 0, -q, q)


def mxfp8_quantize(x: np.ndarray):
    """OCP MXFP8-E4M3 quantization along the last axis (length % 32 == 0):
    per 32 elements the shared scale is X = 2^(floor(log2 amax) - 8) (the E4M3
    largest exponent is 8), held at E8M0's smallest 2^-127 when lower; elements
    are x/X rounded to E4M3 with saturation; an all-zero block gets scale
    exponent 0 (byte 127) and zero elements.
    Returns (element values float64 [..., K], scale exponents int [..., K/32])."""
    x = np.asarray(x, dtype=np.float64)
    shp = x.shape
    blk = x.reshape(-1, shp[-1] // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    e = np.where(np.exp2(e) > amax, e - 1, e)
    e = np.where(np.exp2(e + 1) <= amax, e + 1, e)
    e = np.where(amax > 0, np.maximum(e - 8.0, -127.0), 0.0)
    X = np.exp2(e)
    elems = e4m3_round(blk / X[..., None])
    return elems.reshape(shp), e.astype(np.int64).reshape(shp[:-1] + (shp[-1] // 32,))
