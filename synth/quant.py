"""Fixture encoders: float weights -> routed-expert bytes.

Both encoders are plain min/max (Q2K) or OCP-rule (MXFP4) quantizers written
for test fixtures; they are not an imitation of any library's search.  Only the
bytes they produce matter for parity, because both the oracle and the kernels
start from those bytes.  They run on whatever device the input tensor is on
(CPU for small layers, the GPU for full-size ones).

Q2K-style super-block (84 bytes per 256 consecutive weights of a flat
row-major matrix):
  bytes  0..15  one byte per group j of 16 weights: scale s_j in the low
                nibble, min m_j in the high nibble
  bytes 16..79  2-bit codes, code i (0..255) in byte 16 + i//4 at bits 2*(i%4)
  bytes 80..81  d    (IEEE binary16, little-endian)
  bytes 82..83  dmin (IEEE binary16, little-endian)
and the weight it stands for is d*s_j*q_i - dmin*m_j.  The pages name Q2_K as
the 2-bit super-block format for the routed experts (hysenlabs "DwarfStar実地分析",
section "GGUFの対応範囲は意図的に狭い"; README mirror "DS4 分布式Shell客户端",
section "模型下载"); the exact field order above is this library's choice.

MXFP4 (OCP Microscaling v1.0): per row, K/2 code bytes (element c in byte c//2,
low nibble when c is even; E2M1 nibble = sign<<3 | exp<<1 | mant) followed in a
separate array by K/32 E8M0 scale bytes (scale = 2**(byte-127)).  The pages say
the MXFP4 model keeps DeepSeek's published expert weights (hysenlabs page, same
section); the synthetic weights here stand in for them.
"""
import torch

Q2K_BLOCK = 256
Q2K_BYTES = 84
MX_BLOCK = 32


def q2k_bytes_per_matrix(rows: int, K: int) -> int:
    n = rows * K
    if n % Q2K_BLOCK:
        raise ValueError("rows*K must be a multiple of 256 for Q2K")
    return n // Q2K_BLOCK * Q2K_BYTES


def mxfp4_bytes_per_matrix(rows: int, K: int) -> tuple:
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32 for MXFP4")
    return rows * K // 2, rows * K // MX_BLOCK


def q2k_encode(w: torch.Tensor) -> torch.Tensor:
    """Encode a flat run of weights (any shape, numel % 256 == 0) into Q2K bytes.

    Per group of 16: b = -min(0, min w), a = (max w + b)/3.  Per block:
    d = fp16(max a / 15), dmin = fp16(max b / 15); s = clip(rint(a/d), 0, 15),
    m = clip(rint(b/dmin), 0, 15); q = clip(rint((w + dmin*m)/(d*s)), 0, 3)
    (q = 0 where d*s == 0).  Returns uint8 [numel/256, 84].
    """
    w = w.reshape(-1, 16, 16).to(torch.float32)
    nb = w.shape[0]
    b = (-w.amin(dim=-1)).clamp(min=0.0)                # [nb,16]
    a = (w.amax(dim=-1) + b) / 3.0
    d = (a.amax(dim=-1) / 15.0).to(torch.float16)       # [nb]
    dmin = (b.amax(dim=-1) / 15.0).to(torch.float16)
    df = d.to(torch.float32)[:, None]
    dmf = dmin.to(torch.float32)[:, None]
    zero = torch.zeros_like(a)
    s = torch.where(df > 0, torch.round(a / torch.where(df > 0, df, 1.0)), zero).clamp(0, 15)
    m = torch.where(dmf > 0, torch.round(b / torch.where(dmf > 0, dmf, 1.0)), zero).clamp(0, 15)
    scale = (df * s)[:, :, None]
    mn = (dmf * m)[:, :, None]
    q = torch.where(scale > 0, torch.round((w + mn) / torch.where(scale > 0, scale, 1.0)),
                    torch.zeros_like(w)).clamp(0, 3)
    q = q.to(torch.uint8).reshape(nb, 64, 4)
    out = torch.empty(nb, Q2K_BYTES, dtype=torch.uint8, device=w.device)
    out[:, 0:16] = s.to(torch.uint8) | (m.to(torch.uint8) << 4)
    out[:, 16:80] = q[:, :, 0] | (q[:, :, 1] << 2) | (q[:, :, 2] << 4) | (q[:, :, 3] << 6)
    out[:, 80:82] = d.contiguous().view(torch.uint8).reshape(nb, 2)
    out[:, 82:84] = dmin.contiguous().view(torch.uint8).reshape(nb, 2)
    return out


def _e2m1_code(v: torch.Tensor) -> torch.Tensor:
    """|v| -> E2M1 magnitude code 0..7 (values 0,.5,1,1.5,2,3,4,6), round to
    nearest with ties to the even mantissa, saturating at 6."""
    c = ((v > 0.25).to(torch.uint8) + (v >= 0.75).to(torch.uint8) + (v > 1.25).to(torch.uint8)
         + (v >= 1.75).to(torch.uint8) + (v > 2.5).to(torch.uint8) + (v >= 3.5).to(torch.uint8)
         + (v > 5.0).to(torch.uint8))
    return c


def mxfp4_encode(w: torch.Tensor):
    """Encode a [rows, K] matrix into (codes uint8 [rows, K/2], scales uint8 [rows, K/32]).

    OCP rule: X = 2**(floor(log2 amax) - 2) per 32 elements; elements w/X
    rounded to E2M1 (ties to even, saturate at 6); an all-zero block gets
    scale byte 127 and zero codes.
    """
    rows, K = w.shape
    blk = w.to(torch.float32).reshape(rows, K // MX_BLOCK, MX_BLOCK)
    amax = blk.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                          # amax = f * 2**ex, f in [0.5,1)
    e = torch.where(amax > 0, ex.to(torch.int32) - 1 - 2, torch.zeros_like(ex, dtype=torch.int32))
    e = e.clamp(-127, 127)
    scale = torch.ldexp(torch.ones_like(amax), e.to(torch.float32))
    v = blk / scale[..., None]
    mag = _e2m1_code(v.abs())
    sign = (v < 0).to(torch.uint8) & (mag > 0).to(torch.uint8)
    nib = (sign << 3) | mag
    nib = nib.reshape(rows, K // 2, 2)
    codes = nib[:, :, 0] | (nib[:, :, 1] << 4)
    scales = (e + 127).to(torch.uint8)
    return codes.contiguous(), scales.contiguous()


Q4K_PARAM_BYTES = 20


def q4k_bytes_per_matrix(rows: int, K: int) -> tuple:
    if K % Q2K_BLOCK:
        raise ValueError("K must be a multiple of 256 for Q4K")
    return rows * K // 2, rows * K // Q2K_BLOCK * Q4K_PARAM_BYTES


def q4k_encode(w: torch.Tensor):
    """Encode a [rows, K] matrix (K % 256 == 0) into the Q4K-style arrays
    (codes uint8 [rows, K/2], params uint8 [rows, K/256, 20]).

    The 4-bit analogue of the Q2K quantizer above, per 256-weight super-block
    of a row: per group of 16, b = -min(0, min w), a = (max w + b)/15;
    d = fp16(max a / 15), dmin = fp16(max b / 15); s = clip(rint(a/d), 0, 15),
    m = clip(rint(b/dmin), 0, 15), q = clip(rint((w + dmin*m)/(d*s)), 0, 15)
    (q = 0 where d*s == 0).  Codes: element c of a row in byte c/2, low nibble
    when c is even.  Params per super-block: 16 bytes s | m << 4, then d and
    dmin as little-endian fp16.
    """
    rows, K = w.shape
    if K % Q2K_BLOCK:
        raise ValueError("K must be a multiple of 256 for Q4K")
    nb = rows * K // Q2K_BLOCK
    g = w.to(torch.float32).reshape(nb, 16, 16)
    b = (-g.amin(dim=-1)).clamp(min=0.0)
    a = (g.amax(dim=-1) + b) / 15.0
    d = (a.amax(dim=-1) / 15.0).to(torch.float16)
    dmin = (b.amax(dim=-1) / 15.0).to(torch.float16)
    df = d.to(torch.float32)[:, None]
    dmf = dmin.to(torch.float32)[:, None]
    zero = torch.zeros_like(a)
    s = torch.where(df > 0, torch.round(a / torch.where(df > 0, df, 1.0)), zero).clamp(0, 15)
    m = torch.where(dmf > 0, torch.round(b / torch.where(dmf > 0, dmf, 1.0)), zero).clamp(0, 15)
    scale = (df * s)[:, :, None]
    mn = (dmf * m)[:, :, None]
    q = torch.where(scale > 0, torch.round((g + mn) / torch.where(scale > 0, scale, 1.0)),
                    torch.zeros_like(g)).clamp(0, 15)
    q = q.to(torch.uint8).reshape(rows, K // 2, 2)
    codes = q[:, :, 0] | (q[:, :, 1] << 4)
    params = torch.empty(nb, Q4K_PARAM_BYTES, dtype=torch.uint8, device=w.device)
    params[:, 0:16] = s.to(torch.uint8) | (m.to(torch.uint8) << 4)
    params[:, 16:18] = d.contiguous().view(torch.uint8).reshape(nb, 2)
    params[:, 18:20] = dmin.contiguous().view(torch.uint8).reshape(nb, 2)
    return codes.contiguous(), params.reshape(rows, K // Q2K_BLOCK, Q4K_PARAM_BYTES).contiguous()
