// Decode expert FFN (bf16 path): GEMV kernels that stream each touched
// expert's low-bit weights from HBM once per small group of tokens.
//
// Decode is bound by memory bandwidth on the pages' hardware ("284B MoEを
// 128GBノートPCに詰め込む", section "プリフィル790 t/sが暴く真のボトルネック"),
// and the routed experts dominate the model's bytes (hysenlabs
// "DwarfStar実地分析", section "SSDストリーミングは容量を広げる代わりに
// 速度を譲る").  On MI355X a 2-bit weight arrives every 0.33 B, so the kernel
// has under two VALU instructions per weight to turn codes into products.
//
// Q2K: a group's 16 codes are one dword (code c at bits 2c).  One AND-OR with
// a mask and the bf16 pattern of 128 turns two codes (c, c+8) into the bf16
// pair (128 + 4^p q_c, 128 + 4^p q_{c+8}), p = c mod 3 after the two shifts
// that bring codes 3..7 to bit offsets 0, 2, 4.  The activations are staged
// once per token as the matching pairs x_c * 4^-p (exact in bf16), so that
// v_dot2_f32_bf16 accumulates sum_c q_c x_c + 128 sum_c x_c 4^-p; the second
// term is a per-token constant C_g, subtracted by starting the accumulator
// at -C_g (staged negated).  Per group the result is scaled once: d*s*Q - dmin*m*S, with
// S = sum of the group's activations.  About 1.5 VALU instructions/weight.
//
// MXFP4: gfx950's v_cvt_scalef32_pk_bf16_fp4 converts one code byte into a
// bf16 pair exactly; v_dot2_f32_bf16 does the products; the E8M0 scale is
// applied once per 32-element block.
//
// Lane layout: each output row is owned by LPR consecutive lanes (LPR divides
// 16); a lane walks units (Q2K: 64 weights = 4 groups; MXFP4: 32 weights =
// one block) at stride LPR, so the LPR lanes of a row read adjacent 16-byte
// pieces.  A wave holds 64/LPR rows; lanes with the same position in their
// row read the same staged activations (an LDS broadcast).  Staged activations
// are stored piece-major so that consecutive lanes read consecutive 16 bytes.
#include "formats.hpp"
#include "launch.hpp"
#include "vecdot.hpp"

namespace ds4 {

constexpr int GV_TOKC_MAX = 8;    // max tokens per LDS chunk
constexpr int GV_UB = 8;      // units loaded per batch (MXFP4, bf16)
constexpr int GV_UB_Q2K = 4;  // units loaded per batch (Q2K)
struct GvGeom {
    int K, rows, NU, LPR, UPL, tiles, rows_per_tile;  // routed matrices
    int passes;                                        // wave passes (rows_per_tile each) per routed item
    int Ks, rows_s, tiles_s, rows_s_item;              // shared expert (tiles_s = 0: none)
    int tokc;
};

// ---- routed row dots ---------------------------------------------------------
// y[t] += this lane's share of row r of a Q2K matrix times token t's staged
// activations, for t < nt.
template <int TOKC>
__device__ __forceinline__ void q2k_row(const uint8_t* __restrict__ base, int r, const GvGeom& g, int lir,
                                        const uint8_t* lds, int nt, float* y) {
    const int NG = g.K / 16, NQ = g.NU;
    const int64_t fq0 = (int64_t)r * NQ;
    for (int u0 = 0; u0 < g.UPL; u0 += GV_UB_Q2K) {
        u32x4 cw[GV_UB_Q2K];
        uint32_t sd[GV_UB_Q2K], dd[GV_UB_Q2K];
#pragma unroll
        for (int i = 0; i < GV_UB_Q2K; ++i) {
            if (u0 + i < g.UPL) {
                const int64_t fq = fq0 + lir + (int64_t)(u0 + i) * g.LPR;
                const uint8_t* blk = base + (fq >> 2) * Q2K_BLOCK_BYTES;
                const int jq = (int)(fq & 3);
                cw[i] = *reinterpret_cast<const u32x4*>(blk + 16 + 16 * jq);
                sd[i] = ld_u32(blk + 4 * jq);
                dd[i] = ld_u32(blk + 80);
            }
        }
#pragma unroll
        for (int i = 0; i < GV_UB_Q2K; ++i)
            if (u0 + i < g.UPL) q2k_unit_dot<TOKC>(cw[i], sd[i], dd[i], lir + (u0 + i) * g.LPR, lds, NQ, NG, nt, y);
    }
}

// y[t] += this lane's share of row r of a Q4K matrix (codes, 20-byte
// super-block parameters) times token t's staged activations, t < nt.  A
// unit is 64 weights: 32 code bytes, four groups, whose four s|m bytes are
// one dword of the unit's parameter record.
template <int TOKC>
__device__ __forceinline__ void q4k_row(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ params, int r,
                                        const GvGeom& g, int lir, const uint8_t* lds, int nt, float* y) {
    const int NG = g.K / 16, NQ = g.NU;
    const int64_t fq0 = (int64_t)r * NQ;
    // units in flight per batch: twice Q2K's code bytes per unit, so fewer
    // units once several tokens' sums are live (register pressure)
    constexpr int UB = TOKC == 1 ? GV_UB_Q2K : GV_UB_Q2K / 2;
    for (int u0 = 0; u0 < g.UPL; u0 += UB) {
        u32x4 c0[UB], c1[UB];
        uint32_t sd[UB], dd[UB];
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            if (u0 + i < g.UPL) {
                const int64_t fq = fq0 + lir + (int64_t)(u0 + i) * g.LPR;
                const u32x4* cp = reinterpret_cast<const u32x4*>(codes + fq * 32);
                c0[i] = cp[0];
                c1[i] = cp[1];
                const uint8_t* rec = params + (fq >> 2) * Q4K_PARAM_BYTES;
                sd[i] = ld_u32(rec + 4 * (int)(fq & 3));
                dd[i] = ld_u32(rec + 16);
            }
        }
#pragma unroll
        for (int i = 0; i < UB; ++i)
            if (u0 + i < g.UPL)
                q4k_unit_dot<TOKC>(c0[i], c1[i], sd[i], dd[i], lir + (u0 + i) * g.LPR, lds, NQ, NG, nt, y);
    }
}

template <int TOKC>
__device__ __forceinline__ void mx_row(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int r,
                                       const GvGeom& g, int lir, const uint8_t* lds, int nt, float* y) {
    const int NB = g.NU;
    const int64_t fb0 = (int64_t)r * NB;
    for (int u0 = 0; u0 < g.UPL; u0 += GV_UB) {
        u32x4 cw[GV_UB];
        uint32_t sc[GV_UB];
#pragma unroll
        for (int i = 0; i < GV_UB; ++i) {
            if (u0 + i < g.UPL) {
                const int64_t fb = fb0 + lir + (int64_t)(u0 + i) * g.LPR;
                cw[i] = *reinterpret_cast<const u32x4*>(codes + fb * 16);
                sc[i] = scales[fb];
            }
        }
#pragma unroll
        for (int i = 0; i < GV_UB; ++i)
            if (u0 + i < g.UPL) mx_unit_dot<TOKC>(cw[i], sc[i], lir + (u0 + i) * g.LPR, lds, NB, nt, y);
    }
}

// Shared-expert (bf16 weights) row dot over a whole wave: lane l takes
// 8-element chunks l, l+64, ...
template <int TOKC>
__device__ __forceinline__ void bf16_row(const uint16_t* __restrict__ w, int K, int lane, const uint8_t* lds, int nt,
                                         float* y) {
    const int NC = K / 8;
    const u32x4* wr = reinterpret_cast<const u32x4*>(w);
    for (int c0 = 0; c0 < NC; c0 += WAVE * GV_UB) {
        u32x4 wv[GV_UB];
#pragma unroll
        for (int i = 0; i < GV_UB; ++i) {
            const int c = c0 + lane + WAVE * i;
            if (c < NC) wv[i] = wr[c];
        }
#pragma unroll
        for (int i = 0; i < GV_UB; ++i) {
            const int c = c0 + lane + WAVE * i;
            if (c < NC) bf16_chunk_dot<TOKC>(wv[i], c, lds, NC, nt, y);
        }
    }
}

template <int FMT, bool UP, int TOKC>
__global__ __launch_bounds__(256, 2) void gemv_kernel(FfnArgs a, GvGeom g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n_active = active_count(a.active, a.E, a.T * a.k);
    const int routed_items = n_active * g.tiles;
    const int total = routed_items + g.tiles_s;
    const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* hg = reinterpret_cast<const uint16_t*>(a.h);
    const uint16_t* shg = reinterpret_cast<const uint16_t*>(a.sh_h);
    // Shared-expert items first: they are the longest, so they start at once
    // instead of trailing behind the routed ones.
    for (int item0 = blockIdx.x; item0 < total; item0 += gridDim.x) {
        if (item0 >= g.tiles_s) {
            const int item = item0 - g.tiles_s;
            const int e = a.active[1 + item / g.tiles];
            const int rt = item % g.tiles;
            int row0, ntok;
            if (!expert_rows(a.offsets, e, a.E, a.T * a.k, row0, ntok)) continue;
            const size_t ds = expert_data_stride(FMT, g.rows, g.K);
            const size_t ss = expert_scale_stride(FMT, g.rows, g.K);
            const uint8_t* m0 = (UP ? a.gate : a.down) + e * ds;
            const uint8_t* m1 = UP ? a.up + e * ds : nullptr;
            const uint8_t* s0 = FMT != 1 ? (UP ? a.gate_s : a.down_s) + e * ss : nullptr;
            const uint8_t* s1 = (FMT != 1 && UP) ? a.up_s + e * ss : nullptr;
            const int lir = lane % g.LPR;
            for (int c0 = 0; c0 < ntok; c0 += g.tokc) {
                const int nt = min(g.tokc, ntok - c0);
                __syncthreads();
                auto row = [&](int ti) -> const uint16_t* {
                    if (UP) return xg + (size_t)(a.sorted_pair[row0 + c0 + ti] / a.k) * a.H;
                    return hg + (size_t)(row0 + c0 + ti) * a.F;
                };
                if (FMT == WFMT_Q2K) stage_q2k(lds, nt, g.K, row);
                else if (FMT == WFMT_Q4K) stage_q4k(lds, nt, g.K, row);
                else stage_mx(lds, nt, g.K, row);
                __syncthreads();
                for (int ps = 0; ps < g.passes; ++ps) {
                const int r = (rt * g.passes + ps) * g.rows_per_tile + wave * (WAVE / g.LPR) + lane / g.LPR;
                const bool live = r < g.rows;
                float y0[TOKC], y1[TOKC];
#pragma unroll
                for (int t = 0; t < TOKC; ++t) { y0[t] = 0.0f; y1[t] = 0.0f; }
                if (live) {
                    if (FMT == WFMT_Q2K) {
                        q2k_row<TOKC>(m0, r, g, lir, lds, nt, y0);
                        if (UP) q2k_row<TOKC>(m1, r, g, lir, lds, nt, y1);
                    } else if (FMT == WFMT_Q4K) {
                        q4k_row<TOKC>(m0, s0, r, g, lir, lds, nt, y0);
                        if (UP) q4k_row<TOKC>(m1, s1, r, g, lir, lds, nt, y1);
                    } else {
                        mx_row<TOKC>(m0, s0, r, g, lir, lds, nt, y0);
                        if (UP) mx_row<TOKC>(m1, s1, r, g, lir, lds, nt, y1);
                    }
                }
#pragma unroll
                for (int t = 0; t < TOKC; ++t) {
                    if (t < nt) {
                        const float v0 = group_sum(y0[t], g.LPR);
                        const float v1 = UP ? group_sum(y1[t], g.LPR) : 0.0f;
                        if (live && lir == 0) {
                            if (UP)
                                reinterpret_cast<uint16_t*>(a.h)[(size_t)(row0 + c0 + t) * a.F + r] =
                                    (uint16_t)f32_to_bf16(silu_f32(v0) * v1);
                            else
                                reinterpret_cast<uint16_t*>(a.expert_out)[(size_t)(row0 + c0 + t) * a.H + r] =
                                    (uint16_t)f32_to_bf16(v0);
                        }
                    }
                }
                }
            }
        } else {
            const int rt = item0;
            const int ntok = a.T;
            for (int c0 = 0; c0 < ntok; c0 += g.tokc) {
                const int nt = min(g.tokc, ntok - c0);
                __syncthreads();
                auto row = [&](int ti) -> const uint16_t* {
                    if (UP) return xg + (size_t)(c0 + ti) * a.H;
                    return shg + (size_t)(c0 + ti) * a.Fs;
                };
                stage_plain(lds, nt, g.Ks, row);
                __syncthreads();
                for (int rr = 0; rr < g.rows_s_item / 4; ++rr) {
                    const int r = rt * g.rows_s_item + wave * (g.rows_s_item / 4) + rr;
                    if (r >= g.rows_s) break;                  // uniform per wave
                    float y0[TOKC], y1[TOKC];
#pragma unroll
                    for (int t = 0; t < TOKC; ++t) { y0[t] = 0.0f; y1[t] = 0.0f; }
                    if (UP) {
                        bf16_row<TOKC>(a.sh_gate + (size_t)r * g.Ks, g.Ks, lane, lds, nt, y0);
                        bf16_row<TOKC>(a.sh_up + (size_t)r * g.Ks, g.Ks, lane, lds, nt, y1);
                    } else {
                        bf16_row<TOKC>(a.sh_down + (size_t)r * g.Ks, g.Ks, lane, lds, nt, y0);
                    }
#pragma unroll
                    for (int t = 0; t < TOKC; ++t) {
                        if (t < nt) {
                            const float v0 = wave_sum(y0[t]);
                            const float v1 = UP ? wave_sum(y1[t]) : 0.0f;
                            if (lane == 0) {
                                if (UP)
                                    reinterpret_cast<uint16_t*>(a.sh_h)[(size_t)(c0 + t) * a.Fs + r] =
                                        (uint16_t)f32_to_bf16(silu_f32(v0) * v1);
                                else
                                    reinterpret_cast<uint16_t*>(a.shared_out)[(size_t)(c0 + t) * a.H + r] =
                                        (uint16_t)f32_to_bf16(v0);
                            }
                        }
                    }
                }
            }
        }
    }
}

static int gcd16(int n) {
    int l = 16;
    while (l > 1 && n % l) l >>= 1;
    return l;
}

template <int FMT, bool UP>
static hipError_t launch_one(const FfnArgs& a, bool routed, bool shared, hipStream_t s) {
    GvGeom g;
    g.K = UP ? a.H : a.F;
    g.rows = UP ? a.F : a.H;
    g.NU = g.K / (FMT == WFMT_MX ? 32 : 64);
    g.LPR = gcd16(g.NU);
    g.UPL = g.NU / g.LPR;
    g.rows_per_tile = 4 * (WAVE / g.LPR);
    // routed items of ~40-80 KB of weights: one wave pass for the long up
    // rows, several for the short down rows (one LDS staging per item)
    const double row_bytes = FMT == WFMT_Q2K ? g.K / 256.0 * 84
                             : (FMT == WFMT_Q4K ? g.K / 256.0 * 148 : g.K / 2.0 + g.K / 32.0);
    g.passes = 1;
    while (g.passes < 8 && row_bytes * g.rows_per_tile * g.passes * (UP ? 2 : 1) < 40000.0) g.passes *= 2;
    const int rows_per_item = g.rows_per_tile * g.passes;
    g.tiles = routed ? (g.rows + rows_per_item - 1) / rows_per_item : 0;
    g.Ks = UP ? a.H : a.Fs;
    g.rows_s = UP ? a.Fs : a.H;
    // shared items of about the same size: one row (pair) per wave for long rows
    g.rows_s_item = (g.Ks * 2 * (UP ? 2 : 1) * 16 > 160000) ? 4 : 16;
    g.tiles_s = shared ? (g.rows_s + g.rows_s_item - 1) / g.rows_s_item : 0;
    const size_t per_tok_routed = FMT == WFMT_Q2K ? (size_t)(g.K / 16) * 40
                                  : (FMT == WFMT_Q4K ? (size_t)(g.K / 16) * 36 : (size_t)g.K * 2);
    const size_t per_tok_shared = shared ? (size_t)g.Ks * 2 : 0;
    const size_t per_tok = per_tok_routed > per_tok_shared ? per_tok_routed : per_tok_shared;
    // tokens per LDS chunk: a power of two, LDS <= 64 KiB, no more than needed
    int cap = (int)(65536 / per_tok);
    const int need = a.T;
    int tokc = 1;
    while (tokc * 2 <= GV_TOKC_MAX && tokc * 2 <= cap && tokc < need) tokc *= 2;
    g.tokc = tokc;
    const int P = a.T * a.k;
    const int max_active = routed ? (a.E < P ? a.E : P) : 0;
    const int items = max_active * g.tiles + g.tiles_s;
    if (items == 0) return hipSuccess;
    const int grid = items < 2048 ? items : 2048;
    const size_t lds = per_tok * tokc;
    const int stage = UP ? STAGE_FFN_UP : STAGE_FFN_DOWN;
    switch (tokc) {
        case 1: return launch_stage(stage, gemv_kernel<FMT, UP, 1>, dim3(grid), dim3(256), lds, s, a, g);
        case 2: return launch_stage(stage, gemv_kernel<FMT, UP, 2>, dim3(grid), dim3(256), lds, s, a, g);
        case 4: return launch_stage(stage, gemv_kernel<FMT, UP, 4>, dim3(grid), dim3(256), lds, s, a, g);
        default: return launch_stage(stage, gemv_kernel<FMT, UP, 8>, dim3(grid), dim3(256), lds, s, a, g);
    }
}

hipError_t launch_ffn_gemv_bf16(const FfnArgs& a, bool routed, bool shared, hipStream_t s) {
    hipError_t err;
    if (a.wfmt == WFMT_Q2K) {
        err = launch_one<1, true>(a, routed, shared, s);
        return err != hipSuccess ? err : launch_one<1, false>(a, routed, shared, s);
    }
    if (a.wfmt == WFMT_Q4K) {
        err = launch_one<4, true>(a, routed, shared, s);
        return err != hipSuccess ? err : launch_one<4, false>(a, routed, shared, s);
    }
    err = launch_one<2, true>(a, routed, shared, s);
    return err != hipSuccess ? err : launch_one<2, false>(a, routed, shared, s);
}

}  // namespace ds4
