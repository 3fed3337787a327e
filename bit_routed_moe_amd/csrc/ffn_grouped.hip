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

// ---- LDS carve-up ----------------------------------------------------------------
// [0, 2*GG_BUF): double-buffered token tiles.  After them a 3-deep ring of raw
// routed-weight bytes for one stage, each wave writing and reading only its
// own 64 rows, 64 bytes per row.  Consecutive DMA lanes fetch consecutive
// bytes of one row (a few cache lines per instruction).  Within a row the
// 16-byte slots are XOR-swizzled by bits 2..3 of the row, so the 16 rows a
// lane quarter reads hit 16 different bank groups.
//   Q2K dwords: 0..7 the codes of the stage's 8 groups, 8..9 their scale
//   bytes, 10 d|dmin (11..15 unused); dword d sits at slot-swizzled position
//   d ^ (4 * ((row >> 2) & 3)).
//   MXFP4: 4 x 16 B of codes (slot c at c ^ ((row >> 2) & 3)); the rows' E8M0
//   scale dwords follow the 256 code rows.
constexpr int GG_ABUF_Q2K = 256 * 64;
constexpr int GG_ABUF_MX = 256 * 64 + 256 * 4;
constexpr int GG_LDS_Q2K = 2 * GG_BUF + 3 * GG_ABUF_Q2K;
constexpr int GG_LDS_MX = 2 * GG_BUF + 3 * GG_ABUF_MX;

__device__ __forceinline__ int gg_swz(int rr) { return (rr >> 2) & 3; }

__device__ __forceinline__ void gg_dma4(const void* g, const uint8_t* lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds_dst);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, off"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
}

template <typename V>
__device__ __forceinline__ V lds_ld(const uint8_t* p) {
    return *reinterpret_cast<const V*>(p);
}

// bf16 shared-expert rows: loaded straight into registers one stage ahead.
struct GgBf16Raw {
    u32x4 v[4][4];   // [row tile][k-step]
};

__device__ __forceinline__ bf16x8 gg_pack8(const float (&w)[8]) {
    u32x4 v;
    v[0] = pack_bf16x2(w[0], w[1]);
    v[1] = pack_bf16x2(w[2], w[3]);
    v[2] = pack_bf16x2(w[4], w[5]);
    v[3] = pack_bf16x2(w[6], w[7]);
    return __builtin_bit_cast(bf16x8, v);
}

// Decode of the A operands of k-steps 2*gi, 2*gi+1 for one row tile, split
// into an LDS load (issued early) and NS small slices of VALU work that the
// phase loop spreads between matrix instructions (in slice order).  The
// results: r[0] = k-step 2*gi, r[1] = k-step 2*gi+1.
// Pin a value to this point of the instruction stream: an empty volatile asm
// that reads and rewrites it, so the code computing it cannot drift past the
// surrounding scheduling fences (it emits no instruction).
template <typename V>
__device__ __forceinline__ void gg_pin(V& v) {
    asm volatile("" : "+v"(v));
}

template <int KIND>
struct GgDec;

template <>
struct GgDec<GG_KIND_Q2K> {
    static constexpr int NS = 6;
    uint32_t c, scw, dd, x[4];
    float ds9, ndm;
    u32x4 r[2];
    __device__ __forceinline__ void load(const uint8_t* ab, int rr, int q4, int gi) {
        const uint8_t* row = ab + rr * 64;
        const int sw = 4 * gg_swz(rr);
        c = lds_ld<uint32_t>(row + 4 * ((2 * q4 + gi) ^ sw));
        scw = lds_ld<uint32_t>(row + 4 * ((8 + (q4 >> 1)) ^ sw));
        dd = lds_ld<uint32_t>(row + 4 * (10 ^ sw));
    }
    // (x[i] holds code 4j + i in byte j; fp8 word 0 of x[i] -> codes (i, i+4),
    // word 1 -> (i+8, i+12); the fp8 byte q is the subnormal q * 2^-9)
    template <int H, int P>
    __device__ __forceinline__ void quad() {
        const auto pa = __builtin_amdgcn_cvt_pk_f32_fp8(x[2 * P], H != 0);
        const auto pb = __builtin_amdgcn_cvt_pk_f32_fp8(x[2 * P + 1], H != 0);
        uint32_t lo = pack_bf16x2(fmaf(ds9, pa[0], ndm), fmaf(ds9, pb[0], ndm));   // codes 8H+2P, +1
        uint32_t hi = pack_bf16x2(fmaf(ds9, pa[1], ndm), fmaf(ds9, pb[1], ndm));   // codes 8H+2P+4, +5
        gg_pin(lo);
        gg_pin(hi);
        r[H][P] = lo;
        r[H][P + 2] = hi;
    }
    template <int J>
    __device__ __forceinline__ void slice(int q4, int gi) {
        if constexpr (J == 0) {
            const uint32_t sc = (scw >> (8 * (2 * (q4 & 1) + gi))) & 0xFFu;
            const float d = half_bits_to_f32(dd & 0xFFFFu);
            const float dmin = half_bits_to_f32(dd >> 16);
            ds9 = d * (float)(sc & 15u) * 512.0f;     // d*s*2^9, exact
            ndm = -(dmin * (float)(sc >> 4));         // -dmin*m, exact
            gg_pin(ds9);
            gg_pin(ndm);
        } else if constexpr (J == 1) {
            const uint32_t M = 0x03030303u;
            x[0] = c & M;
            x[1] = (c >> 2) & M;
            x[2] = (c >> 4) & M;
            x[3] = (c >> 6) & M;
            gg_pin(x[0]);
            gg_pin(x[1]);
            gg_pin(x[2]);
            gg_pin(x[3]);
        } else if constexpr (J == 2) {
            quad<0, 0>();
        } else if constexpr (J == 3) {
            quad<0, 1>();
        } else if constexpr (J == 4) {
            quad<1, 0>();
        } else {
            quad<1, 1>();
        }
    }
};

template <>
struct GgDec<GG_KIND_MX> {
    static constexpr int NS = 3;
    u32x2 cw;
    uint32_t e;
    float scale;
    u32x4 r[2];
    __device__ __forceinline__ void load(const uint8_t* ab, int rr, int q4, int gi) {
        cw = lds_ld<u32x2>(ab + rr * 64 + 16 * (q4 ^ gg_swz(rr)) + 8 * gi);
        e = ab[256 * 64 + rr * 4 + q4];
    }
    template <int J>
    __device__ __forceinline__ void slice(int, int) {
        if constexpr (J == 0) {
            scale = __uint_as_float(e << 23);   // 2^(e-127)
            gg_pin(scale);
        } else {
            const uint32_t c = cw[J - 1];
            uint32_t v0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0));
            uint32_t v1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1));
            uint32_t v2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2));
            uint32_t v3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3));
            gg_pin(v0);
            gg_pin(v1);
            gg_pin(v2);
            gg_pin(v3);
            r[J - 1][0] = v0;
            r[J - 1][1] = v1;
            r[J - 1][2] = v2;
            r[J - 1][3] = v3;
        }
    }
};

template <int KIND>
__device__ __forceinline__ void gg_slice(GgDec<KIND>& d, int j, int q4, int gi) {
    if constexpr (KIND == GG_KIND_Q2K) {
        switch (j) {
            case 0: d.template slice<0>(q4, gi); break;
            case 1: d.template slice<1>(q4, gi); break;
            case 2: d.template slice<2>(q4, gi); break;
            case 3: d.template slice<3>(q4, gi); break;
            case 4: d.template slice<4>(q4, gi); break;
            default: d.template slice<5>(q4, gi); break;
        }
    } else {
        switch (j) {
            case 0: d.template slice<0>(q4, gi); break;
            case 1: d.template slice<1>(q4, gi); break;
            default: d.template slice<2>(q4, gi); break;
        }
    }
}

// One phase: the MFMAs of k-steps s0, s0+1 for all token tiles (each B
// fragment feeds the 4 row tiles), software-pipelined in source order: B
// fragments are read two tile-steps ahead, and when DEC the decode slices of
// the next operands (group gi_dec of the stage staged at ab_dec) are spread
// evenly over the tile-steps.  Each step is fenced (sched_barrier) and laid
// out as MFMA, VALU share, MFMA, ... so the matrix core and the VALU overlap
// with one wave per SIMD.
template <int KIND, int NT, bool DEC>
__device__ __forceinline__ void gg_phase(f32x4 (&acc)[4][NT], const bf16x8 (&A)[4][2], const uint8_t* bb, int q4,
                                         int m, int s0, const uint8_t* ab_dec, int rr0, int gi_dec,
                                         bf16x8 (&D)[4][2]) {
    constexpr int STEPS = 2 * NT;
    constexpr int DK = KIND == GG_KIND_BF16 ? GG_KIND_MX : KIND;
    constexpr int NS = GgDec<DK>::NS;
    constexpr int NSL = 4 * NS;                                   // slices per phase
    constexpr int VALU_PER_SLICE = KIND == GG_KIND_Q2K ? 8 : 4;
    constexpr int VPM = DEC ? (NSL * VALU_PER_SLICE + 4 * STEPS - 1) / (4 * STEPS) : 0;
    GgDec<DK> dec[4];
    if constexpr (DEC) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dec[rt].load(ab_dec, rr0 + 16 * rt, q4, gi_dec);
    }
    auto bread = [&](int i) {
        const int ss = i / NT, t = i % NT;
        const int slot = ((4 * q4 + s0 + ss) ^ m) << 4;
        return lds_ld<bf16x8>(bb + t * GG_TT * GG_ROWB + slot);
    };
    bf16x8 b0 = bread(0);
    bf16x8 b1 = STEPS > 1 ? bread(1) : b0;
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        bf16x8 b2 = b1;
        if (i + 2 < STEPS) b2 = bread(i + 2);
        const int ss = i / NT, t = i % NT;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rt][ss], b0, acc[rt][t], 0, 0, 0);
        if constexpr (DEC) {
#pragma unroll
            for (int q = 0; q < NSL; ++q)
                if ((q * STEPS) / NSL == i) gg_slice<DK>(dec[q / NS], q % NS, q4, gi_dec);
        }
        if constexpr (DEC) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);   // VALU
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // DS read
        }
        __builtin_amdgcn_sched_barrier(0);
        b0 = b1;
        b1 = b2;
    }
    if constexpr (DEC) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            D[rt][0] = __builtin_bit_cast(bf16x8, dec[rt].r[0]);
            D[rt][1] = __builtin_bit_cast(bf16x8, dec[rt].r[1]);
        }
    }
}

// ---- one work unit ---------------------------------------------------------------
// NT = token tiles of the chunk (compile time, so the tile loops are straight
// line code that the scheduler can pipeline).
template <int KIND, bool UP, int NT>
__device__ __forceinline__ void gg_unit(const GgArgs& a, const GgChunk& ch, int rb, uint8_t* lds) {
    constexpr bool SH = KIND == GG_KIND_BF16;
    constexpr int ABUF = KIND == GG_KIND_Q2K ? GG_ABUF_Q2K : GG_ABUF_MX;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m = lane & 15, q4 = lane >> 4;
    const int K = SH ? a.Ks : a.K;
    const int nst = K / GG_KS;
    const int n = ch.n;

    // Weight row of WG row rr = 64*w + 16*rt + mm: up: rt 0,1 -> gate rows
    // f0 + 16*rt + mm, rt 2,3 -> up rows f0 + 16*(rt-2) + mm (f0 = rb*128 +
    // 32*w); down: row rb*256 + rr.
    auto wrow = [&](int rt, int mm) {
        return UP ? rb * 128 + 32 * w + 16 * (rt & 1) + mm : rb * 256 + 64 * w + 16 * rt + mm;
    };
    auto wmat = [&](int rt) -> const uint8_t* {
        if (SH) return reinterpret_cast<const uint8_t*>(UP && rt >= 2 ? a.sw1 : a.sw0);
        return (UP && rt >= 2 ? a.w1 : a.w0) + (size_t)ch.expert * a.wstride;
    };

    // Raw-weight DMA.  Q2K: instruction j of this wave fills WG rows 64*w +
    // 4*j .. +3 (row tile j/4), lane l -> row + (l >> 4), LDS dword slot
    // l & 15 = field (l & 15) ^ (4 * (j & 3)).  MXFP4: instruction j fills rows
    // 64*w + 16*j .. +15, lane l -> row + (l >> 2), slot l & 3 = chunk
    // (l & 3) ^ ((l >> 4) & 3); one more dword instruction per wave fetches
    // its 64 rows' scales (lane = row).
    uint8_t* abase = lds + 2 * GG_BUF;
    auto stage_a = [&](int st) {
        uint8_t* ab = abase + (st % 3) * ABUF + 64 * w * 64;
        if constexpr (KIND == GG_KIND_Q2K) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rt = j >> 2;
                const int64_t row = wrow(rt, 4 * (j & 3) + (lane >> 4));
                const int64_t fg = row * (K / 16) + 8 * st;     // first group of the stage: 0 or 8 in its block
                const uint8_t* blk = wmat(rt) + (fg >> 4) * 84;
                const int g0 = (int)(fg & 15);
                const int d = (lane & 15) ^ (4 * (j & 3));
                const int off = d < 8 ? 16 + 4 * (g0 + d) : (d < 10 ? g0 + 4 * (d - 8) : 80);
                gg_dma4(blk + off, ab + j * 256);
            }
        } else if constexpr (KIND == GG_KIND_MX) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = wrow(j, lane >> 2);
                const int c = (lane & 3) ^ ((lane >> 4) & 3);
                gg_dma16(wmat(j) + row * (K / 2) + 64 * st + 16 * c, ab + j * 1024);
            }
            const int rt = lane >> 4;
            const int64_t row = wrow(rt, lane & 15);
            const uint8_t* sc = (UP && rt >= 2 ? a.s1 : a.s0) + (size_t)ch.expert * a.sstride + row * (K / 32);
            gg_dma4(sc + 4 * st, abase + (st % 3) * ABUF + 256 * 64 + 64 * w * 4);
        }
    };

    // bf16 rows of the consumer lanes (shared expert)
    const uint8_t* brow[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) brow[rt] = SH ? wmat(rt) + (size_t)wrow(rt, m) * K * 2 + 64 * q4 : nullptr;
    auto load_bf16 = [&](GgBf16Raw& r, int st) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int s = 0; s < 4; ++s) r.v[rt][s] = *reinterpret_cast<const u32x4*>(brow[rt] + 256 * st + 16 * s);
    };

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
    auto stage_x = [&](int st) {
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

    const int rr0 = 64 * w + m;   // + 16*rt: this lane's consumer rows
    if constexpr (SH) {
        GgBf16Raw cur, nxt;
        stage_x(0);
        load_bf16(cur, 0);
        for (int st = 0; st < nst; ++st) {
            gg_wait_all();
            __syncthreads();
            if (st + 1 < nst) {
                stage_x(st + 1);
                load_bf16(nxt, st + 1);
            }
            const uint8_t* bb = lds + (st & 1) * GG_BUF + m * GG_ROWB;
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                bf16x8 A[4][2], unused[4][2];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    A[rt][0] = __builtin_bit_cast(bf16x8, cur.v[rt][2 * gi]);
                    A[rt][1] = __builtin_bit_cast(bf16x8, cur.v[rt][2 * gi + 1]);
                }
                gg_phase<KIND, NT, false>(acc, A, bb, q4, m, 2 * gi, nullptr, 0, 0, unused);
            }
            if (st + 1 < nst) cur = nxt;
        }
    } else {
        // Raw bytes of stage st+2 and token rows of stage st+1 are staged at
        // the top of stage st and waited for at its end.  Phase 0 runs stage
        // st's k-steps 0,1 on the matrix cores while the VALUs decode its
        // second group; phase 1 runs k-steps 2,3 while they decode the first
        // group of stage st+1 (on the last stage a stale buffer, unused), so
        // each phase is one straight-line block the scheduler can interleave.
        stage_x(0);
        stage_a(0);
        if (nst > 1) stage_a(1);
        gg_wait_all();
        __syncthreads();
        bf16x8 Ag[4][2], Ah[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            GgDec<KIND> d0;
            d0.load(abase, rr0 + 16 * rt, q4, 0);
#pragma unroll
            for (int j = 0; j < GgDec<KIND>::NS; ++j) gg_slice<KIND>(d0, j, q4, 0);
            Ag[rt][0] = __builtin_bit_cast(bf16x8, d0.r[0]);
            Ag[rt][1] = __builtin_bit_cast(bf16x8, d0.r[1]);
        }
        for (int st = 0; st < nst; ++st) {
            if (st + 1 < nst) stage_x(st + 1);
            if (st + 2 < nst) stage_a(st + 2);
            const uint8_t* ab = abase + (st % 3) * ABUF;
            const uint8_t* abn = abase + ((st + 1) % 3) * ABUF;
            const uint8_t* bb = lds + (st & 1) * GG_BUF + m * GG_ROWB;
            gg_phase<KIND, NT, true>(acc, Ag, bb, q4, m, 0, ab, rr0, 1, Ah);
            gg_phase<KIND, NT, true>(acc, Ah, bb, q4, m, 2, abn, rr0, 0, Ag);
            gg_wait_all();
            __syncthreads();
        }
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
    __shared__ __attribute__((aligned(1024))) uint8_t lds[FMT == 1 ? GG_LDS_Q2K : GG_LDS_MX];
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
