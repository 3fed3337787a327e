// Device decode of the routed-expert weight formats.  Every kernel that reads
// routed or shared weights, and the dequantize test export, goes through the
// routines here, so a weight has one device value everywhere.
//
// Q2K-style super-block (84 B per 256 consecutive weights of an expert's flat
// row-major matrix): bytes 0..15 hold group j's 4-bit scale s_j (low nibble)
// and 4-bit min m_j (high nibble); bytes 16..79 the 2-bit codes, code i at
// bits 2*(i%4) of byte 16 + i/4 -- so group j's 16 codes are exactly the
// little-endian dword at byte 16 + 4j, code c of the group at bits 2c; bytes
// 80..83 are d and dmin as fp16.  Weight = d*s_j*q - dmin*m_j.  The pages name
// Q2_K super-blocks for the routed experts (hysenlabs "DwarfStar実地分析",
// section "GGUFの対応範囲は意図的に狭い"); this field order is the library's.
//
// Exactness: d*s (<= 15 significant bits) and d*s*q (<= 17) and dmin*m are
// exact in fp32, so fmaf(d*s, q, -dmin*m) rounds the exact weight once: the
// device fp32 weight is the exact value rounded to nearest fp32, and every
// non-zero weight is a multiple of 2^-24, far from fp32 subnormals.
//
// MXFP4 (OCP MX v1.0): E2M1 nibbles (sign, 2-bit exponent, 1-bit mantissa),
// element c of a row in byte c/2 (low nibble for even c), one E8M0 scale
// 2^(s-127) per 32 elements.  E2M1 * 2^k is exact in fp32 (subnormal results
// included: fp32 denormals are kept on this target).
#pragma once
#include "common.hpp"

namespace ds4 {

constexpr int Q2K_BLOCK_BYTES = 84;

struct Q2KGroup {
    uint32_t codes;   // 16 x 2-bit codes, code c at bits 2c
    float a;          // d * s
    float b;          // dmin * m
};

// Group G (16 consecutive flat weights) of a Q2K matrix starting at `base`.
__device__ __forceinline__ Q2KGroup q2k_load_group(const uint8_t* base, int64_t G) {
    const uint8_t* blk = base + (G >> 4) * Q2K_BLOCK_BYTES;
    const int g = (int)(G & 15);
    const uint32_t sm = blk[g];
    const uint32_t dd = ld_u32(blk + 80);
    Q2KGroup r;
    r.codes = ld_u32(blk + 16 + 4 * g);
    r.a = half_bits_to_f32(dd & 0xFFFFu) * (float)(sm & 15u);
    r.b = half_bits_to_f32(dd >> 16) * (float)(sm >> 4);
    return r;
}

// Weight c (0..15) of a decoded group, rounded once to fp32.
__device__ __forceinline__ float q2k_weight(const Q2KGroup& g, int c) {
    return fmaf(g.a, (float)((g.codes >> (2 * c)) & 3u), -g.b);
}

// Q4K-style super-block (the 4-bit analogue of the block above, 148 B per
// 256 weights of a row, in two arrays): codes [rows][K/2], element c of a row
// in byte c/2 (low nibble for even c, q = 0..15), and per 256 weights of a
// row one 20-byte parameter record: bytes 0..15 s_j | m_j << 4 of group j,
// bytes 16..19 d and dmin as fp16.  Weight = d*s_j*q - dmin*m_j.  The pages
// name 4-bit expert files (README mirror "DS4 分布式Shell客户端", section
// "模型下载") without a layout; this one is the library's.  Exactness as for
// Q2K: d*s (<= 15 significant bits), d*s*q (<= 19) and dmin*m are exact in
// fp32, so fmaf(d*s, q, -dmin*m) rounds the exact weight once.
constexpr int Q4K_PARAM_BYTES = 20;

// Weight c (0..15) of group G (flat weights 16G .. 16G+15) of a Q4K matrix
// (whole super-blocks per row, so flat group G is in record G / 16).
__device__ __forceinline__ void q4k_group_f32(const uint8_t* codes, const uint8_t* params, int64_t G, float w[16]) {
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes + G * 8);
    const uint8_t* rec = params + (G >> 4) * Q4K_PARAM_BYTES;
    const uint32_t sm = rec[G & 15];
    const uint32_t dd = ld_u32(rec + 16);
    const float a = half_bits_to_f32(dd & 0xFFFFu) * (float)(sm & 15u);
    const float b = half_bits_to_f32(dd >> 16) * (float)(sm >> 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t c = cw[h];
#pragma unroll
        for (int n = 0; n < 8; ++n) w[8 * h + n] = fmaf(a, (float)((c >> (4 * n)) & 15u), -b);
    }
}

// E2M1 nibble -> value (exact).  2*|v| for codes 0..7 is 0,1,2,3,4,6,8,12.
__device__ __forceinline__ float e2m1_value(uint32_t nib) {
    const uint64_t twice = 0x0C08060403020100ull;
    const float mag = (float)((twice >> (8 * (nib & 7u))) & 0xFFu) * 0.5f;
    return (nib & 8u) ? -mag : mag;
}

__device__ __forceinline__ float e8m0_scale(uint32_t s) {
    return ldexpf(1.0f, (int)s - 127);
}

// Weight (flat index f) of an MXFP4 matrix: value * scale (exact in fp32).
__device__ __forceinline__ float mxfp4_weight(const uint8_t* codes, const uint8_t* scales, int64_t f) {
    const uint32_t byte = codes[f >> 1];
    const uint32_t nib = (f & 1) ? (byte >> 4) : (byte & 15u);
    return ldexpf(e2m1_value(nib), (int)scales[f >> 5] - 127);
}

// MXFP8-E4M3 (OCP MX v1.0) activation blocks: 32 consecutive values share
// the E8M0 scale 2^(floor(log2 amax) - 8) (8 = E4M3's largest exponent),
// held no lower than E8M0's 2^-127; an all-zero block takes 2^0.  Elements
// are value / scale rounded to nearest-even E4M3 (OCP, bias 7), saturating at
// +-448.  The pages' 8-bit activation packing is an E4M3-like f8 (qiita
// "DwarfStar の TCP パイプライン分散推論を読む", section 9); the block scaling
// is OCP MX's.
//
// Scale byte of a block from its largest magnitude: the biased fp32 exponent
// of amax is floor(log2 amax) + 127 for normal amax, so the E8M0 byte is that
// minus 8 (a subnormal amax lands below 0 and is held at 0).
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
    if (!(amax > 0.0f)) return 127u;
    const int e = (int)(__float_as_uint(amax) >> 23) - 8;
    return e < 0 ? 0u : (uint32_t)e;
}

// 1 / scale = 2^(127 - byte), a normal fp32 for every byte mx8_scale_byte
// returns; value * (1 / scale) is exact (|result| < 2^9).
__device__ __forceinline__ float mx8_inv_scale(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }

// Four scaled values -> four E4M3 bytes (value j in byte j): clamp to +-448,
// then one nearest-even conversion (v_cvt_pk_fp8_f32), which equals rounding
// first and saturating after.
__device__ __forceinline__ uint32_t mx8_pack4(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    c = fminf(fmaxf(c, -448.0f), 448.0f);
    d = fminf(fmaxf(d, -448.0f), 448.0f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// Decode 16 consecutive weights of group G (flat weights 16G .. 16G+15) of a
// matrix in format `wfmt` (1 Q2K, 2 MXFP4, 3 BF16, 4 Q4K) to fp32.
__device__ __forceinline__ void decode_group_f32(int wfmt, const uint8_t* data, const uint8_t* scales,
                                                 int64_t G, float w[16]) {
    if (wfmt == 4) {
        q4k_group_f32(data, scales, G, w);
    } else if (wfmt == 1) {
        const Q2KGroup g = q2k_load_group(data, G);
#pragma unroll
        for (int c = 0; c < 16; ++c) w[c] = q2k_weight(g, c);
    } else if (wfmt == 2) {
        const uint32_t* cw = reinterpret_cast<const uint32_t*>(data + G * 8);
        const uint32_t c0 = cw[0], c1 = cw[1];
        const int sc = (int)scales[G >> 1] - 127;
#pragma unroll
        for (int c = 0; c < 8; ++c) w[c] = ldexpf(e2m1_value((c0 >> (4 * c)) & 15u), sc);
#pragma unroll
        for (int c = 0; c < 8; ++c) w[8 + c] = ldexpf(e2m1_value((c1 >> (4 * c)) & 15u), sc);
    } else {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(data + G * 32);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t v = p[c];
            w[2 * c] = bf16_to_f32(v & 0xFFFFu);
            w[2 * c + 1] = bf16_to_f32(v >> 16);
        }
    }
}

}  // namespace ds4
