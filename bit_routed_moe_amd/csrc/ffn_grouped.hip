// Prefill expert FFN (bf16 path): grouped GEMM on the matrix cores.
//
// With thousands of tokens per call every routed expert sees on the order of a
// hundred tokens, so each dequantized weight feeds a hundred multiply-adds and
// the work is a dense contraction: "DS4 分布式Shell客户端" (README mirror,
// section on the distributed prefill) splits prompts into 4096-token chunks,
// and "284B MoEを128GBノートPCに詰め込む" (section on the 790 t/s prefill)
// places the batched-expert work on matrix instructions.  Here it runs on
// gfx950's v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// Work unit: one workgroup (4 waves) computes a 128-row (up: gate + up rows of
// 128 ffn columns) or 256-row (down) block of one matrix for one chunk of at
// most 192 tokens of one expert.  A one-workgroup plan kernel lists the chunks
// (experts with more than 192 tokens are split evenly, in 16-token granules).
//
// Operands, per 16x16x32 MFMA: A = 16 weight rows x 32 reduction columns,
// B = 32 columns x 16 tokens.  Lane l holds row/token (l % 16) and columns
// 8*(l/16) .. +7 of the step.  Each wave owns 4 row tiles (64 rows), so every
// B fragment read from LDS feeds 4 MFMAs, and each weight is dequantized
// exactly once per workgroup, into registers.  Per 128-column stage the lane
// quarter q (= l/16) owns reduction columns 32q .. 32q+31, which is two whole
// 16-weight Q2K groups (one scale byte each), one 32-weight MXFP4 block (one
// E8M0 scale), or 64 contiguous bytes of a bf16 row.
//
// Weight decode ("DwarfStar実地分析", section on the intentionally narrow GGUF
// support: the 2-bit routed experts; OCP MX for MXFP4):
//   Q2K   w = RN_bf16(fmaf(d*s, q, -dmin*m)); the 2-bit codes are spread into
//         bytes with masks and converted by v_cvt_pk_f32_fp8 (an fp8 byte
//         0..3 is the subnormal q * 2^-9, so multiplying by d*s*2^9 restores
//         d*s*q exactly).
//   MXFP4 v_cvt_scalef32_pk_bf16_fp4 with the E8M0 scale as fp32 exponent:
//         exact.
//   bf16  (shared expert) loaded as is.
//
// Token rows (x for up, the SwiGLU output h for down) are staged per stage
// into a double-buffered LDS tile by global_load_lds_dwordx4 (1 KiB per wave
// instruction: 4 token rows x 256 B); 16-byte slots are XOR-swizzled by the
// row's low 4 bits so the B reads are free of bank conflicts.
//
// Outputs are bf16: h = silu(gate) * up rows [P][F] in sorted pair order
// (shared: [T][Fs]); expert_out [P][H] (shared_out [T][H]).
#include "common.hpp"
#include "launch.hpp"

namespace ds4 {

namespace {

constexpr int GG_TT = 16;                     // tokens per MFMA tile
constexpr int GG_NT = 12;                     // token tiles per chunk
constexpr int GG_CT = GG_TT * GG_NT;          // tokens per chunk (192)
constexpr int GG_KS = 128;                    // reduction columns per LDS stage
constexpr int GG_ROWB = GG_KS * 2;            // bytes per staged token row
constexpr int GG_BUF = GG_CT * GG_ROWB;       // one stage buffer: 48 KiB
constexpr int GG_KIND_Q2K = 1, GG_KIND_MX = 2, GG_KIND_BF16 = 3;

struct GgChunk {
    int32_t expert;   // routed expert id, or E for the shared expert
    int32_t row0;     // first sorted pair row (routed) or first token (shared)
    int32_t n;        // tokens in the chunk, 1 .. GG_CT
    int32_t pad;
};

struct GgArgs {
    int E, k, P, T;
    int K, Ks;              // reduction length: routed, shared
    int rows, rows_s;       // rows of one matrix: routed, shared
    int RB;                 // row blocks per chunk in the grid
    const GgChunk* chunks;
    const int32_t* n_chunks;
    const int32_t* sorted_pair;
    const uint8_t *w0, *w1;        // routed data: up: gate, up; down: down
    const uint8_t *s0, *s1;        // MXFP4 scales (same roles)
    const uint16_t *sw0, *sw1;     // shared bf16 matrices (same roles)
    const uint16_t* b;             // routed B rows: up x [T][H]; down h [P][F]
    const uint16_t* bs;            // shared B rows: up x [T][H]; down sh_h [T][Fs]
    int ldb, ldbs;                 // their row lengths (elements)
    uint16_t* out;                 // up: h [P][F]; down: expert_out [P][H]
    uint16_t* outs;                // up: sh_h [T][Fs]; down: shared_out [T][H]
    int ldo, ldos;
    size_t wstride, sstride;       // routed per-expert data / scale strides (bytes)
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---- chunk plan ----------------------------------------------------------------
// One 1024-thread workgroup: thread e lists the chunks of expert e (those with
// min_tok <= n_e <= max_tok); the shared expert's chunks come first.
__global__ __launch_bounds__(1024) void gg_plan_kernel(const int32_t* __restrict__ offsets, int E, int P, int T,
                                                     int min_tok, int max_tok, int routed, int shared,
                                                     GgChunk* __restrict__ chunks, int32_t* __restrict__ n_chunks,
                                                     int cmax) {
    __shared__ int tmp[32];
    const int e = threadIdx.x;
    int n = 0, nch = 0;
    if (routed && e < E) {
        const int r0 = offsets[e], r1 = offsets[e + 1];
        n = r1 - r0;
        if (r0 < 0 || r1 > P || n < 0) n = 0;
        if (n < min_tok || n > max_tok) n = 0;
        nch = ceil_div(n, GG_CT);
    }
    const int nsh = shared ? ceil_div(T, GG_CT) : 0;
    int total;
    const int base = nsh + block_exclusive_scan(nch, tmp, &total);
    total += nsh;
    if (total > cmax) total = 0;   // cannot happen for a valid permutation
    if (total == 0) {
        if (e == 0) n_chunks[0] = 0;
        return;
    }
    auto emit = [&](int c0, int expert, int row0, int cnt, int pieces) {
        const int cs = ceil_div(ceil_div(cnt, pieces), GG_TT) * GG_TT;
        for (int i = 0; i < pieces; ++i) {
            GgChunk c;
            c.expert = expert;
            c.row0 = row0 + i * cs;
            c.n = min(cs, cnt - i * cs);
            c.pad = 0;
            chunks[c0 + i] = c;
        }
    };
    if (nch > 0) emit(base, e, offsets[e], n, nch);
    if (e == 0) {
        if (nsh > 0) emit(0, E, 0, T, nsh);
        n_chunks[0] = total;
    }
}

// ---- LDS DMA -------------------------------------------------------------------
// 64 lanes x 16 B from global memory into LDS at lds_dst + 16*lane.  Issued as
// inline asm so that the compiler's wait-count pass does not make every later
// LDS read wait for all outstanding loads; the stage loop waits explicitly.
__device__ __forceinline__ void gg_dma16(const void* g, const uint8_t* lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds_dst);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
}

__device__ __forceinline__ void gg_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- per-kind weight fragments -------------------------------------------------
// Raw bytes one lane loads per stage for its 4 row tiles, and their decode into
// the A operands of the stage's 4 k-steps (two at a time).
template <int KIND>
struct GgRaw;

template <>
struct GgRaw<GG_KIND_Q2K> {
    uint32_t c0[4], c1[4], sc[4], dd[4];
};
template <>
struct GgRaw<GG_KIND_MX> {
    u32x4 c[4];
    uint32_t e[4];
};
template <>
struct GgRaw<GG_KIND_BF16> {
    u32x4 v[4][4];
};

// Where row tile rt of this lane reads: Q2K keeps the flat group index of the
// lane's first group at stage 0 (a matrix is a flat run of 256-weight blocks,
// so a row may start inside a block); MXFP4 keeps code and scale row bases;
// bf16 keeps the row base.
struct GgRowPtr {
    const uint8_t* data;
    const uint8_t* scale;
    int64_t fg;
};

template <int KIND>
__device__ __forceinline__ void gg_load(GgRaw<KIND>& r, const GgRowPtr (&p)[4], int st) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        if constexpr (KIND == GG_KIND_Q2K) {
            const int64_t fg = p[rt].fg + 8 * st;                 // even: both groups in one block
            const uint8_t* blk = p[rt].data + (fg >> 4) * 84;
            const int g = (int)(fg & 15);
            r.c0[rt] = ld_u32(blk + 16 + 4 * g);
            r.c1[rt] = ld_u32(blk + 20 + 4 * g);
            r.sc[rt] = *reinterpret_cast<const uint16_t*>(blk + g);
            r.dd[rt] = ld_u32(blk + 80);
        } else if constexpr (KIND == GG_KIND_MX) {
            r.c[rt] = *reinterpret_cast<const u32x4*>(p[rt].data + 64 * st);
            r.e[rt] = p[rt].scale[4 * st];
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) r.v[rt][s] = *reinterpret_cast<const u32x4*>(p[rt].data + 256 * st + 16 * s);
        }
    }
}

__device__ __forceinline__ bf16x8 gg_pack8(const float (&w)[8]) {
    u32x4 v;
    v[0] = pack_bf16x2(w[0], w[1]);
    v[1] = pack_bf16x2(w[2], w[3]);
    v[2] = pack_bf16x2(w[4], w[5]);
    v[3] = pack_bf16x2(w[6], w[7]);
    return __builtin_bit_cast(bf16x8, v);
}

// A operands of k-steps 2*gi and 2*gi+1 for row tile rt.
template <int KIND>
__device__ __forceinline__ void gg_decode(const GgRaw<KIND>& r, int rt, int gi, bf16x8& a0, bf16x8& a1) {
    if constexpr (KIND == GG_KIND_Q2K) {
        const uint32_t c = gi == 0 ? r.c0[rt] : r.c1[rt];
        const uint32_t sc = (r.sc[rt] >> (8 * gi)) & 0xFFu;
        const float d = half_bits_to_f32(r.dd[rt] & 0xFFFFu);
        const float dmin = half_bits_to_f32(r.dd[rt] >> 16);
        const float ds9 = d * (float)(sc & 15u) * 512.0f;     // d*s*2^9, exact
        const float ndm = -(dmin * (float)(sc >> 4));         // -dmin*m, exact
        const uint32_t M = 0x03030303u;
        // byte j of cj holds code 4*j' + i for the shift i: (c >> 2i) & M
        const uint32_t x0 = c & M, x1 = (c >> 2) & M, x2 = (c >> 4) & M, x3 = (c >> 6) & M;
        // fp8 words: lo -> codes (i, i+4), hi -> codes (i+8, i+12)
        const auto p0l = __builtin_amdgcn_cvt_pk_f32_fp8(x0, false), p0h = __builtin_amdgcn_cvt_pk_f32_fp8(x0, true);
        const auto p1l = __builtin_amdgcn_cvt_pk_f32_fp8(x1, false), p1h = __builtin_amdgcn_cvt_pk_f32_fp8(x1, true);
        const auto p2l = __builtin_amdgcn_cvt_pk_f32_fp8(x2, false), p2h = __builtin_amdgcn_cvt_pk_f32_fp8(x2, true);
        const auto p3l = __builtin_amdgcn_cvt_pk_f32_fp8(x3, false), p3h = __builtin_amdgcn_cvt_pk_f32_fp8(x3, true);
        float w0[8], w1[8];
        w0[0] = fmaf(ds9, p0l[0], ndm); w0[4] = fmaf(ds9, p0l[1], ndm);
        w0[1] = fmaf(ds9, p1l[0], ndm); w0[5] = fmaf(ds9, p1l[1], ndm);
        w0[2] = fmaf(ds9, p2l[0], ndm); w0[6] = fmaf(ds9, p2l[1], ndm);
        w0[3] = fmaf(ds9, p3l[0], ndm); w0[7] = fmaf(ds9, p3l[1], ndm);
        w1[0] = fmaf(ds9, p0h[0], ndm); w1[4] = fmaf(ds9, p0h[1], ndm);
        w1[1] = fmaf(ds9, p1h[0], ndm); w1[5] = fmaf(ds9, p1h[1], ndm);
        w1[2] = fmaf(ds9, p2h[0], ndm); w1[6] = fmaf(ds9, p2h[1], ndm);
        w1[3] = fmaf(ds9, p3h[0], ndm); w1[7] = fmaf(ds9, p3h[1], ndm);
        a0 = gg_pack8(w0);
        a1 = gg_pack8(w1);
    } else if constexpr (KIND == GG_KIND_MX) {
        const float scale = __uint_as_float(r.e[rt] << 23);   // 2^(e-127)
        const uint32_t ca = r.c[rt][2 * gi], cb = r.c[rt][2 * gi + 1];
        u32x4 v0, v1;
        v0[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ca, scale, 0));
        v0[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ca, scale, 1));
        v0[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ca, scale, 2));
        v0[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ca, scale, 3));
        v1[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cb, scale, 0));
        v1[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cb, scale, 1));
        v1[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cb, scale, 2));
        v1[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cb, scale, 3));
        a0 = __builtin_bit_cast(bf16x8, v0);
        a1 = __builtin_bit_cast(bf16x8, v1);
    } else {
        a0 = __builtin_bit_cast(bf16x8, r.v[rt][2 * gi]);
        a1 = __builtin_bit_cast(bf16x8, r.v[rt][2 * gi + 1]);
    }
}

// ---- one work unit ---------------------------------------------------------------
// NT = token tiles of the chunk (compile time, so the tile loops are straight
// line code that the scheduler can pipeline).
template <int KIND, bool UP, int NT>
__device__ __forceinline__ void gg_unit(const GgArgs& a, const GgChunk& ch, int rb, uint8_t* lds) {
    constexpr bool SH = KIND == GG_KIND_BF16;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m = lane & 15, q4 = lane >> 4;
    const int K = SH ? a.Ks : a.K;
    const int nst = K / GG_KS;
    const int n = ch.n;

    // weight rows of this lane's 4 row tiles
    GgRowPtr rp[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        int row;
        const uint8_t* mat;
        const uint8_t* smat = nullptr;
        if (UP) {
            row = rb * 128 + 32 * w + 16 * (rt & 1) + m;
            if (SH) {
                mat = reinterpret_cast<const uint8_t*>(rt < 2 ? a.sw0 : a.sw1);
            } else {
                mat = (rt < 2 ? a.w0 : a.w1) + (size_t)ch.expert * a.wstride;
                if (KIND == GG_KIND_MX) smat = (rt < 2 ? a.s0 : a.s1) + (size_t)ch.expert * a.sstride;
            }
        } else {
            row = rb * 256 + 64 * w + 16 * rt + m;
            if (SH) {
                mat = reinterpret_cast<const uint8_t*>(a.sw0);
            } else {
                mat = a.w0 + (size_t)ch.expert * a.wstride;
                if (KIND == GG_KIND_MX) smat = a.s0 + (size_t)ch.expert * a.sstride;
            }
        }
        if constexpr (KIND == GG_KIND_Q2K) {
            rp[rt].data = mat;
            rp[rt].scale = nullptr;
            rp[rt].fg = (int64_t)row * (K / 16) + 2 * q4;
        } else if constexpr (KIND == GG_KIND_MX) {
            rp[rt].data = mat + (size_t)row * (K / 2) + 16 * q4;
            rp[rt].scale = smat + (size_t)row * (K / 32) + q4;
            rp[rt].fg = 0;
        } else {
            rp[rt].data = mat + (size_t)row * K * 2 + 64 * q4;
            rp[rt].scale = nullptr;
            rp[rt].fg = 0;
        }
    }

    // token rows this lane stages: row r_in of every tile, 16-byte slot col
    const int r_in = 4 * w + (lane >> 4);
    const int col = (lane & 15) ^ r_in;
    const uint16_t* bsrc = SH ? a.bs : a.b;
    const int ldb = SH ? a.ldbs : a.ldb;
    int32_t ridx[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        int i = 16 * j + r_in;
        if (i > n - 1) i = n - 1;
        int r;
        if (UP && !SH) {
            r = a.sorted_pair[ch.row0 + i] / a.k;
            if ((unsigned)r >= (unsigned)a.T) r = 0;   // corrupt permutation: stay in bounds
        } else {
            r = ch.row0 + i;
        }
        ridx[j] = r;
    }
    auto stage_in = [&](int st) {
        const uint8_t* dst = lds + (st & 1) * GG_BUF;
#pragma unroll
        for (int j = 0; j < NT; ++j)
            gg_dma16(bsrc + (size_t)ridx[j] * ldb + st * GG_KS + 8 * col, dst + (w + 4 * j) * 1024);
    };

    f32x4 acc[4][NT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    GgRaw<KIND> cur, nxt;
    stage_in(0);
    gg_load<KIND>(cur, rp, 0);
    for (int st = 0; st < nst; ++st) {
        gg_wait_all();
        __syncthreads();
        if (st + 1 < nst) {
            stage_in(st + 1);
            gg_load<KIND>(nxt, rp, st + 1);
        }
        const uint8_t* bb = lds + (st & 1) * GG_BUF + m * GG_ROWB;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            bf16x8 A0[4], A1[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) gg_decode<KIND>(cur, rt, gi, A0[rt], A1[rt]);
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
                const int s = 2 * gi + ss;
                const int slot = ((4 * q4 + s) ^ m) << 4;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8*>(bb + t * GG_TT * GG_ROWB + slot);
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
                        acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ss ? A1[rt] : A0[rt], b, acc[rt][t],
                                                                             0, 0, 0);
                }
            }
        }
        if (st + 1 < nst) cur = nxt;
    }

    // epilogue: lane holds rows 4*q4 + i of each row tile for token 16t + m
    uint16_t* out = SH ? a.outs : a.out;
    const int ldo = SH ? a.ldos : a.ldo;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int i = 16 * t + m;
        if (i < n) {
            uint16_t* orow = out + (size_t)(ch.row0 + i) * ldo;
            if (UP) {
                const int f0 = rb * 128 + 32 * w + 4 * q4;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    u32x2 v;
                    v[0] = pack_bf16x2(silu_f32(acc[h][t][0]) * acc[2 + h][t][0],
                                       silu_f32(acc[h][t][1]) * acc[2 + h][t][1]);
                    v[1] = pack_bf16x2(silu_f32(acc[h][t][2]) * acc[2 + h][t][2],
                                       silu_f32(acc[h][t][3]) * acc[2 + h][t][3]);
                    *reinterpret_cast<u32x2*>(orow + f0 + 16 * h) = v;
                }
            } else {
                const int c0 = rb * 256 + 64 * w + 4 * q4;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    u32x2 v;
                    v[0] = pack_bf16x2(acc[rt][t][0], acc[rt][t][1]);
                    v[1] = pack_bf16x2(acc[rt][t][2], acc[rt][t][3]);
                    *reinterpret_cast<u32x2*>(orow + c0 + 16 * rt) = v;
                }
            }
        }
    }
}

template <int KIND, bool UP>
__device__ __forceinline__ void gg_dispatch(const GgArgs& a, const GgChunk& ch, int rb, uint8_t* lds, int nt) {
    switch (nt) {
        case 1: gg_unit<KIND, UP, 1>(a, ch, rb, lds); break;
        case 2: gg_unit<KIND, UP, 2>(a, ch, rb, lds); break;
        case 3: gg_unit<KIND, UP, 3>(a, ch, rb, lds); break;
        case 4: gg_unit<KIND, UP, 4>(a, ch, rb, lds); break;
        case 5: gg_unit<KIND, UP, 5>(a, ch, rb, lds); break;
        case 6: gg_unit<KIND, UP, 6>(a, ch, rb, lds); break;
        case 7: gg_unit<KIND, UP, 7>(a, ch, rb, lds); break;
        case 8: gg_unit<KIND, UP, 8>(a, ch, rb, lds); break;
        case 9: gg_unit<KIND, UP, 9>(a, ch, rb, lds); break;
        case 10: gg_unit<KIND, UP, 10>(a, ch, rb, lds); break;
        case 11: gg_unit<KIND, UP, 11>(a, ch, rb, lds); break;
        default: gg_unit<KIND, UP, 12>(a, ch, rb, lds); break;
    }
}

// Grid: RB row blocks x (chunks padded to a multiple of 8).  The hardware
// deals workgroups to the 8 XCDs round-robin, so workgroup b runs on XCD b % 8;
// chunk c is placed on XCD c % 8 and its RB row blocks are dealt to that XCD
// back to back: they share the chunk's token rows in the XCD's L2.
template <int FMT, bool UP>
__global__ __launch_bounds__(256, 1) void gg_kernel(GgArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * GG_BUF];
    const int bid = blockIdx.x;
    const int j = bid >> 3;
    const int chunk = (j / a.RB) * 8 + (bid & 7);
    const int rb = j % a.RB;
    if (chunk >= a.n_chunks[0]) return;
    const GgChunk ch = a.chunks[chunk];
    const bool shared = ch.expert == a.E;
    if (ch.n < 1 || ch.n > GG_CT || ch.row0 < 0 || (!shared && (ch.expert < 0 || ch.expert > a.E))) return;
    if (ch.row0 + ch.n > (shared ? a.T : a.P)) return;
    const int rows = shared ? a.rows_s : a.rows;
    if ((rb + 1) * (UP ? 128 : 256) > rows) return;
    const int nt = (ch.n + GG_TT - 1) / GG_TT;
    if (shared)
        gg_dispatch<GG_KIND_BF16, UP>(a, ch, rb, lds, nt);
    else
        gg_dispatch<FMT, UP>(a, ch, rb, lds, nt);
}

int gg_max_chunks(int E, int P, int T, bool routed, bool shared) {
    int c = 0;
    if (routed) c += (E < P ? E : P) + P / GG_CT + 1;
    if (shared) c += (T + GG_CT - 1) / GG_CT;
    return c;
}

template <int FMT, bool UP>
hipError_t gg_launch(const FfnArgs& f, const GgChunk* chunks, const int32_t* n_chunks, int cmax, bool routed,
                     bool shared, hipStream_t s) {
    GgArgs a;
    a.E = f.E;
    a.k = f.k;
    a.T = f.T;
    a.P = f.T * f.k;
    a.K = UP ? f.H : f.F;
    a.Ks = UP ? f.H : f.Fs;
    a.rows = UP ? f.F : f.H;
    a.rows_s = UP ? f.Fs : f.H;
    const int rbr = routed ? (UP ? f.F / 128 : f.H / 256) : 0;
    const int rbs = shared ? (UP ? f.Fs / 128 : f.H / 256) : 0;
    a.RB = rbr > rbs ? rbr : rbs;
    a.chunks = chunks;
    a.n_chunks = n_chunks;
    a.sorted_pair = f.sorted_pair;
    a.w0 = UP ? f.gate : f.down;
    a.w1 = UP ? f.up : nullptr;
    a.s0 = UP ? f.gate_s : f.down_s;
    a.s1 = UP ? f.up_s : nullptr;
    a.sw0 = UP ? f.sh_gate : f.sh_down;
    a.sw1 = UP ? f.sh_up : nullptr;
    a.b = UP ? static_cast<const uint16_t*>(f.x) : static_cast<const uint16_t*>(f.h);
    a.bs = UP ? static_cast<const uint16_t*>(f.x) : static_cast<const uint16_t*>(f.sh_h);
    a.ldb = UP ? f.H : f.F;
    a.ldbs = UP ? f.H : f.Fs;
    a.out = UP ? static_cast<uint16_t*>(f.h) : static_cast<uint16_t*>(f.expert_out);
    a.outs = UP ? static_cast<uint16_t*>(f.sh_h) : static_cast<uint16_t*>(f.shared_out);
    a.ldo = UP ? f.F : f.H;
    a.ldos = UP ? f.Fs : f.H;
    a.wstride = expert_data_stride(FMT, UP ? f.F : f.H, UP ? f.H : f.F);
    a.sstride = expert_scale_stride(UP ? f.F : f.H, UP ? f.H : f.F);
    const int cpad = (cmax + 7) / 8 * 8;
    const long long grid = (long long)cpad * a.RB;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    return launch_stage(UP ? STAGE_FFN_UP : STAGE_FFN_DOWN, gg_kernel<FMT, UP>, dim3((unsigned)grid), dim3(256), 0, s,
                        a);
}

}  // namespace

size_t grouped_plan_bytes(int E, int T, int k, bool shared) {
    const long long P = (long long)T * k;
    const int c = gg_max_chunks(E, (int)P, T, true, shared);
    return 256 + (size_t)c * sizeof(GgChunk);
}

hipError_t launch_ffn_grouped_bf16(const FfnArgs& f, bool routed, bool shared, hipStream_t s) {
    if (!routed && !shared) return hipSuccess;
    const int P = f.T * f.k;
    const int cmax = gg_max_chunks(f.E, P, f.T, routed, shared);
    int32_t* n_chunks = f.plan;
    GgChunk* chunks = reinterpret_cast<GgChunk*>(reinterpret_cast<uint8_t*>(f.plan) + 256);
    hipLaunchKernelGGL(gg_plan_kernel, dim3(1), dim3(1024), 0, s, f.offsets, f.E, P, f.T, f.min_tokens, f.max_tokens,
                       routed ? 1 : 0, shared ? 1 : 0, chunks, n_chunks, cmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (f.wfmt == 1) {
        e = gg_launch<1, true>(f, chunks, n_chunks, cmax, routed, shared, s);
        if (e != hipSuccess) return e;
        return gg_launch<1, false>(f, chunks, n_chunks, cmax, routed, shared, s);
    }
    e = gg_launch<2, true>(f, chunks, n_chunks, cmax, routed, shared, s);
    if (e != hipSuccess) return e;
    return gg_launch<2, false>(f, chunks, n_chunks, cmax, routed, shared, s);
}

}  // namespace ds4
