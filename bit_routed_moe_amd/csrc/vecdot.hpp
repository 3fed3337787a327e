// Dot-product building blocks of the bf16-path GEMV kernels (decode):
// bf16 pair dots, the Q2K code expansion that feeds them without forming
// weight values, the exact E2M1 byte conversion, and the staging of
// activation rows into LDS in the layouts those dots read.
//
// Q2K: a group's 16 codes are one dword (code c at bits 2c).  One AND-OR with
// a mask and the bf16 pattern of 128 turns two codes (c, c+8) into the bf16
// pair (128 + 4^p q_c, 128 + 4^p q_{c+8}), p = c mod 3 after the two shifts
// that bring codes 3..7 to bit offsets 0, 2, 4.  Activations are staged as
// the matching pairs x_c * 4^-p (exact in bf16), so v_dot2_f32_bf16
// accumulates sum_c q_c x_c + 128 sum_c x_c 4^-p; the second term is a
// per-group constant C_g, removed by starting the accumulator at -C_g (staged
// already negated).  Each
// group is then scaled once: d*s*Q - dmin*m*S, S = the group's activation sum.
#pragma once
#include "common.hpp"

namespace ds4 {

constexpr uint32_t BF16_128X2 = 0x43004300u;

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// (a & m) | o in one v_and_or_b32 (m uniform, in an SGPR).  Written out because the compiler otherwise
// splits it into an AND and an OR with literal operands (VOP3 takes no
// literal here), doubling the expansion cost.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
    return r;
}

// Byte B of v as fp32 (v_cvt_f32_ubyteB).
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
    float r;
    if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
    else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
    else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Expansion of a Q2K code dword into the 8 bf16 pairs described above.
__device__ __forceinline__ void q2k_expand(uint32_t c, uint32_t e[8]) {
    const uint32_t k = BF16_128X2, m0 = 0x00030003u, m1 = 0x000C000Cu, m2 = 0x00300030u;
    const uint32_t c6 = c >> 6, c12 = c >> 12;
    e[0] = and_or(c, m0, k);
    e[1] = and_or(c, m1, k);
    e[2] = and_or(c, m2, k);
    e[3] = and_or(c6, m0, k);
    e[4] = and_or(c6, m1, k);
    e[5] = and_or(c6, m2, k);
    e[6] = and_or(c12, m0, k);
    e[7] = and_or(c12, m1, k);
}

// Q4K: a group's 16 codes are two dwords (code c at bits 4(c%8) of dword
// c/8).  One AND-OR of a dword shifted right by 4n with the nibble mask of
// both halves and the bf16 pattern of 128 gives the pair (128 + q_n,
// 128 + q_{n+4}) of the dword's eight codes (a nibble fills the low mantissa
// bits of 128, where the spacing is 1).  Activations are staged as the
// matching pairs (x_n, x_{n+4}), so v_dot2_f32_bf16 accumulates
// sum_c q_c x_c + 128 sum_c x_c; the accumulator starts at -128 S (S = the
// group's activation sum) to remove the second term.
__device__ __forceinline__ void q4k_expand(uint32_t c, uint32_t e[4]) {
    const uint32_t k = BF16_128X2, m = 0x000F000Fu;
    e[0] = and_or(c, m, k);
    e[1] = and_or(c >> 4, m, k);
    e[2] = and_or(c >> 8, m, k);
    e[3] = and_or(c >> 12, m, k);
}

// One byte (two E2M1 codes, low nibble first) -> bf16 pair, exact.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// ---- unit dots -----------------------------------------------------------------
// One lane's unit of a weight row against the staged activations of tokens
// t < nt (layouts below): y[t] += the unit's share of the row dot.

// Q2K unit Qd (64 weights = 4 groups): code quad cw (group q = dword q), the
// four s|m<<4 bytes sd, fp16 d | dmin<<16 dd.
template <int TOKC>
__device__ __forceinline__ void q2k_unit_dot(u32x4 cw, uint32_t sd, uint32_t dd, int Qd, const uint8_t* lds, int NQ,
                                             int NG, int nt, float* y) {
    const u32x4* xq = reinterpret_cast<const u32x4*>(lds);
    const float* C = reinterpret_cast<const float*>(lds + (size_t)nt * NG * 32);
    const float* S = C + nt * NG;
    const float d = half_bits_to_f32(dd & 0xFFFFu);
    const float dmin = half_bits_to_f32(dd >> 16);
    const uint32_t sn = sd & 0x0F0F0F0Fu, mn = (sd >> 4) & 0x0F0F0F0Fu;
    float sf[4], mf[4];
    sf[0] = (float)((sn) & 0xFFu); mf[0] = (float)((mn) & 0xFFu);
    sf[1] = (float)((sn >> 8) & 0xFFu); mf[1] = (float)((mn >> 8) & 0xFFu);
    sf[2] = (float)((sn >> 16) & 0xFFu); mf[2] = (float)((mn >> 16) & 0xFFu);
    sf[3] = (float)((sn >> 24) & 0xFFu); mf[3] = (float)((mn >> 24) & 0xFFu);
    float Pacc[TOKC], Macc[TOKC];
#pragma unroll
    for (int t = 0; t < TOKC; ++t) { Pacc[t] = 0.0f; Macc[t] = 0.0f; }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t e[8];
        q2k_expand(cw[q], e);
#pragma unroll
        for (int t = 0; t < TOKC; ++t) {
            if (t >= nt) break;
            const u32x4 xa = xq[(t * 8 + 2 * q) * NQ + Qd];
            const u32x4 xb = xq[(t * 8 + 2 * q + 1) * NQ + Qd];
            float acc = C[t * NG + 4 * Qd + q];   // -C_g
            acc = dot2bf(e[0], xa[0], acc);
            acc = dot2bf(e[1], xa[1], acc);
            acc = dot2bf(e[2], xa[2], acc);
            acc = dot2bf(e[3], xa[3], acc);
            acc = dot2bf(e[4], xb[0], acc);
            acc = dot2bf(e[5], xb[1], acc);
            acc = dot2bf(e[6], xb[2], acc);
            acc = dot2bf(e[7], xb[3], acc);
            Pacc[t] = fmaf(sf[q], acc, Pacc[t]);
            Macc[t] = fmaf(mf[q], S[t * NG + 4 * Qd + q], Macc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < TOKC; ++t) {
        if (t >= nt) break;
        y[t] = fmaf(d, Pacc[t], y[t]);
        y[t] = fmaf(-dmin, Macc[t], y[t]);
    }
}

// Q4K unit Qd (64 weights = 4 groups): code quads c0 (groups 0, 1) and c1
// (groups 2, 3), the four s|m<<4 bytes sd, fp16 d | dmin<<16 dd.
template <int TOKC>
__device__ __forceinline__ void q4k_unit_dot(u32x4 c0, u32x4 c1, uint32_t sd, uint32_t dd, int Qd, const uint8_t* lds,
                                             int NQ, int NG, int nt, float* y) {
    const u32x4* xq = reinterpret_cast<const u32x4*>(lds);
    const float* S = reinterpret_cast<const float*>(lds + (size_t)nt * NG * 32);
    const float d = half_bits_to_f32(dd & 0xFFFFu);
    const float dmin = half_bits_to_f32(dd >> 16);
    const uint32_t sn = sd & 0x0F0F0F0Fu, mn = (sd >> 4) & 0x0F0F0F0Fu;
    float sf[4], mf[4];
    sf[0] = (float)((sn) & 0xFFu); mf[0] = (float)((mn) & 0xFFu);
    sf[1] = (float)((sn >> 8) & 0xFFu); mf[1] = (float)((mn >> 8) & 0xFFu);
    sf[2] = (float)((sn >> 16) & 0xFFu); mf[2] = (float)((mn >> 16) & 0xFFu);
    sf[3] = (float)((sn >> 24) & 0xFFu); mf[3] = (float)((mn >> 24) & 0xFFu);
    float Pacc[TOKC], Macc[TOKC];
#pragma unroll
    for (int t = 0; t < TOKC; ++t) { Pacc[t] = 0.0f; Macc[t] = 0.0f; }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t e0[4], e1[4];
        q4k_expand(q < 2 ? c0[2 * q] : c1[2 * q - 4], e0);
        q4k_expand(q < 2 ? c0[2 * q + 1] : c1[2 * q - 3], e1);
#pragma unroll
        for (int t = 0; t < TOKC; ++t) {
            if (t >= nt) break;
            const u32x4 xa = xq[(t * 8 + 2 * q) * NQ + Qd];
            const u32x4 xb = xq[(t * 8 + 2 * q + 1) * NQ + Qd];
            const float sg = S[t * NG + 4 * Qd + q];
            float acc = -128.0f * sg;
            acc = dot2bf(e0[0], xa[0], acc);
            acc = dot2bf(e0[1], xa[1], acc);
            acc = dot2bf(e0[2], xa[2], acc);
            acc = dot2bf(e0[3], xa[3], acc);
            acc = dot2bf(e1[0], xb[0], acc);
            acc = dot2bf(e1[1], xb[1], acc);
            acc = dot2bf(e1[2], xb[2], acc);
            acc = dot2bf(e1[3], xb[3], acc);
            Pacc[t] = fmaf(sf[q], acc, Pacc[t]);
            Macc[t] = fmaf(mf[q], sg, Macc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < TOKC; ++t) {
        if (t >= nt) break;
        y[t] = fmaf(d, Pacc[t], y[t]);
        y[t] = fmaf(-dmin, Macc[t], y[t]);
    }
}

// MXFP4 block B (32 weights): code quad cw, E8M0 scale byte sc.
template <int TOKC>
__device__ __forceinline__ void mx_unit_dot(u32x4 cw, uint32_t sc, int B, const uint8_t* lds, int NB, int nt,
                                            float* y) {
    const u32x4* xm = reinterpret_cast<const u32x4*>(lds);
    uint32_t e[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        e[4 * q + 0] = fp4x2_to_bf16x2<0>(cw[q]);
        e[4 * q + 1] = fp4x2_to_bf16x2<1>(cw[q]);
        e[4 * q + 2] = fp4x2_to_bf16x2<2>(cw[q]);
        e[4 * q + 3] = fp4x2_to_bf16x2<3>(cw[q]);
    }
    const int ex = (int)(sc & 0xFFu) - 127;
#pragma unroll
    for (int t = 0; t < TOKC; ++t) {
        if (t >= nt) break;
        float acc = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const u32x4 xa = xm[(t * 4 + v) * NB + B];
            acc = dot2bf(e[4 * v + 0], xa[0], acc);
            acc = dot2bf(e[4 * v + 1], xa[1], acc);
            acc = dot2bf(e[4 * v + 2], xa[2], acc);
            acc = dot2bf(e[4 * v + 3], xa[3], acc);
        }
        y[t] += ldexpf(acc, ex);
    }
}

// bf16 chunk c (8 weights) against plain staged rows [nt][NC] of chunks.
template <int TOKC>
__device__ __forceinline__ void bf16_chunk_dot(u32x4 w, int c, const uint8_t* lds, int NC, int nt, float* y) {
    const u32x4* xs = reinterpret_cast<const u32x4*>(lds);
#pragma unroll
    for (int t = 0; t < TOKC; ++t) {
        if (t >= nt) break;
        const u32x4 xv = xs[t * NC + c];
        float acc = y[t];
        acc = dot2bf(w[0], xv[0], acc);
        acc = dot2bf(w[1], xv[1], acc);
        acc = dot2bf(w[2], xv[2], acc);
        acc = dot2bf(w[3], xv[3], acc);
        y[t] = acc;
    }
}

// ---- staging ---------------------------------------------------------------
// Q2K activation pieces for nt token rows of length K (bf16).  Layout:
//   xq [nt][8][K/64] u32x4 : piece v of quad Q = pairs 4*(v%2).. of group 4Q+v/2
//   C  [nt][K/16] float    : -128 * sum of the group's pre-scaled activations
//   S  [nt][K/16] float    : sum of the group's activations
__device__ __forceinline__ void stage_q2k_group(uint8_t* lds, int nt, int K, int ti, int G, u32x4 lo, u32x4 hi) {
    const int NG = K / 16, NQ = K / 64;
    u32x4* xq = reinterpret_cast<u32x4*>(lds);
    float* C = reinterpret_cast<float*>(lds + (size_t)nt * NG * 32);
    float* S = C + nt * NG;
    float xv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        xv[2 * q] = bf16_to_f32(lo[q] & 0xFFFFu);
        xv[2 * q + 1] = bf16_to_f32(lo[q] >> 16);
        xv[8 + 2 * q] = bf16_to_f32(hi[q] & 0xFFFFu);
        xv[8 + 2 * q + 1] = bf16_to_f32(hi[q] >> 16);
    }
    float ssum = 0.0f, csum = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) ssum += xv[c];
    uint32_t pr[8];
#pragma unroll
    for (int pi = 0; pi < 8; ++pi) {
        const float sc = (pi % 3 == 0) ? 1.0f : ((pi % 3 == 1) ? 0.25f : 0.0625f);
        const float a0 = xv[pi] * sc, a1 = xv[pi + 8] * sc;
        pr[pi] = pack_bf16x2(a0, a1);    // exact: power-of-two scaling of bf16 values
        csum += a0 + a1;
    }
    const int v0 = 2 * (G & 3);
    xq[(ti * 8 + v0) * NQ + (G >> 2)] = u32x4{pr[0], pr[1], pr[2], pr[3]};
    xq[(ti * 8 + v0 + 1) * NQ + (G >> 2)] = u32x4{pr[4], pr[5], pr[6], pr[7]};
    C[ti * NG + G] = -128.0f * csum;
    S[ti * NG + G] = ssum;
}

template <typename RowFn>
__device__ void stage_q2k(uint8_t* lds, int nt, int K, RowFn row) {
    const int NG = K / 16;
    for (int i = threadIdx.x; i < nt * NG; i += blockDim.x) {
        const int ti = i / NG, G = i % NG;
        const u32x4* src = reinterpret_cast<const u32x4*>(row(ti) + 16 * G);
        stage_q2k_group(lds, nt, K, ti, G, src[0], src[1]);
    }
}

// Q4K activation pieces for nt token rows of length K (bf16).  Layout:
//   xq [nt][8][K/64] u32x4 : piece v of unit Q (64 weights) = the pairs
//                            (x_n, x_{n+4}), n = 0..3, of elements 8v .. 8v+7
//   S  [nt][K/16] float    : sum of the group's activations
__device__ __forceinline__ void stage_q4k_group(uint8_t* lds, int nt, int K, int ti, int G, u32x4 lo, u32x4 hi) {
    const int NG = K / 16, NQ = K / 64;
    u32x4* xq = reinterpret_cast<u32x4*>(lds);
    float* S = reinterpret_cast<float*>(lds + (size_t)nt * NG * 32);
    float xv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        xv[2 * q] = bf16_to_f32(lo[q] & 0xFFFFu);
        xv[2 * q + 1] = bf16_to_f32(lo[q] >> 16);
        xv[8 + 2 * q] = bf16_to_f32(hi[q] & 0xFFFFu);
        xv[8 + 2 * q + 1] = bf16_to_f32(hi[q] >> 16);
    }
    float ssum = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) ssum += xv[c];
    const int v0 = 2 * (G & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        u32x4 pc;
#pragma unroll
        for (int n = 0; n < 4; ++n) pc[n] = pack_bf16x2(xv[8 * h + n], xv[8 * h + n + 4]);   // exact: bf16 values
        xq[(ti * 8 + v0 + h) * NQ + (G >> 2)] = pc;
    }
    S[ti * NG + G] = ssum;
}

template <typename RowFn>
__device__ void stage_q4k(uint8_t* lds, int nt, int K, RowFn row) {
    const int NG = K / 16;
    for (int i = threadIdx.x; i < nt * NG; i += blockDim.x) {
        const int ti = i / NG, G = i % NG;
        const u32x4* src = reinterpret_cast<const u32x4*>(row(ti) + 16 * G);
        stage_q4k_group(lds, nt, K, ti, G, src[0], src[1]);
    }
}

// The MXFP4 layout below for one 16-element group G (32 bytes) of row ti.
__device__ __forceinline__ void stage_mx_group(uint8_t* lds, int nt, int K, int ti, int G, u32x4 lo, u32x4 hi) {
    const int NB = K / 32;
    u32x4* xm = reinterpret_cast<u32x4*>(lds);
    const int v0 = 2 * (G & 1);
    xm[(ti * 4 + v0) * NB + (G >> 1)] = lo;
    xm[(ti * 4 + v0 + 1) * NB + (G >> 1)] = hi;
}

// MXFP4 activation pieces: xm [nt][4][K/32] u32x4, piece v of block B = its
// elements 8v .. 8v+7 in natural order.
template <typename RowFn>
__device__ void stage_mx(uint8_t* lds, int nt, int K, RowFn row) {
    const int NB = K / 32;
    u32x4* xm = reinterpret_cast<u32x4*>(lds);
    for (int i = threadIdx.x; i < nt * NB * 4; i += blockDim.x) {
        const int ti = i / (NB * 4), rem = i % (NB * 4);
        const int B = rem >> 2, v = rem & 3;
        xm[(ti * 4 + v) * NB + B] = *reinterpret_cast<const u32x4*>(row(ti) + 32 * B + 8 * v);
    }
}

// Plain bf16 rows [nt][K].
template <typename RowFn>
__device__ void stage_plain(uint8_t* lds, int nt, int K, RowFn row) {
    u32x4* xs = reinterpret_cast<u32x4*>(lds);
    const int NC = K / 8;
    for (int i = threadIdx.x; i < nt * NC; i += blockDim.x) {
        const int ti = i / NC, c = i % NC;
        xs[ti * NC + c] = *reinterpret_cast<const u32x4*>(row(ti) + 8 * c);
    }
}

}  // namespace ds4
