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
//
// A workgroup's routed items run as one software pipeline per wave: two
// batches of units in flight, each requested as the batch two places before
// it is reduced, across the staging barrier and into the next item.
#include "formats.hpp"
#include "launch.hpp"
#include "vecdot.hpp"

namespace ds4 {

constexpr int GV_TOKC_MAX = 8;    // max tokens per LDS chunk
constexpr int GV_UB = 8;          // 16-byte chunks per lane loaded per batch (bf16 shared rows)
struct GvGeom {
    int K, rows, NU, LPR, UPL, tiles, rows_per_tile;  // routed matrices
    int passes;                                        // wave passes (rows_per_tile each) per routed item
    int Ks, rows_s, tiles_s, rows_s_item;              // shared expert (tiles_s = 0: none)
    int tokc;
};

// Routed token rows staged in the layout of the format's unit dot.
template <int FMT, typename RowFn>
__device__ __forceinline__ void stage_routed(uint8_t* lds, int nt, int K, RowFn row) {
    if constexpr (FMT == WFMT_Q2K) stage_q2k(lds, nt, K, row);
    else if constexpr (FMT == WFMT_Q4K) stage_q4k(lds, nt, K, row);
    else stage_mx(lds, nt, K, row);
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

// ---- routed units in flight ---------------------------------------------------
// One unit's registers: Q2K 64 weights of an 84-byte block (code quad, s|m
// dword, d|dmin dword); Q4K 64 weights (two code quads, the parameter
// record's s|m dword and d|dmin dword); MXFP4 one 32-weight block.
template <int FMT>
struct GvUnit;
template <>
struct GvUnit<WFMT_Q2K> {
    u32x4 c;
    uint32_t s, d;
};
template <>
struct GvUnit<WFMT_Q4K> {
    u32x4 c0, c1;
    uint32_t s, d;
};
template <>
struct GvUnit<WFMT_MX> {
    u32x4 c;
    uint32_t s;
};

// Units per batch (a wave keeps two batches in flight): four for MXFP4 (80 B
// per lane); two for Q2K (48 B per lane: against four, 2-8-token steps
// measured 1-2.5% faster and 1-token GEMV steps 8%, the halved registers
// letting more waves share a SIMD; one unit was slower from 6 tokens up);
// two for Q4K with several tokens' sums live (register pressure), else four.
template <int FMT, int TOKC>
constexpr int gv_batch_units() {
    return FMT == WFMT_Q2K ? 2 : (FMT == WFMT_Q4K && TOKC > 1 ? 2 : 4);
}

// Unit fq (row * NU + unit) of a matrix.
template <int FMT>
__device__ __forceinline__ void gv_load(GvUnit<FMT>& u, const uint8_t* __restrict__ m,
                                        const uint8_t* __restrict__ ms, int64_t fq) {
    if constexpr (FMT == WFMT_Q2K) {
        const uint8_t* blk = m + (fq >> 2) * Q2K_BLOCK_BYTES;
        const int jq = (int)(fq & 3);
        u.c = *reinterpret_cast<const u32x4*>(blk + 16 + 16 * jq);
        u.s = ld_u32(blk + 4 * jq);
        u.d = ld_u32(blk + 80);
    } else if constexpr (FMT == WFMT_Q4K) {
        const u32x4* cp = reinterpret_cast<const u32x4*>(m + fq * 32);
        u.c0 = cp[0];
        u.c1 = cp[1];
        const uint8_t* rec = ms + (fq >> 2) * Q4K_PARAM_BYTES;
        u.s = ld_u32(rec + 4 * (int)(fq & 3));
        u.d = ld_u32(rec + 16);
    } else {
        u.c = *reinterpret_cast<const u32x4*>(m + fq * 16);
        u.s = ms[fq];
    }
}

template <int FMT, int TOKC>
__device__ __forceinline__ void gv_dot(const GvUnit<FMT>& u, int Qd, const uint8_t* lds, int NU, int NG, int nt,
                                       float* y) {
    if constexpr (FMT == WFMT_Q2K) q2k_unit_dot<TOKC>(u.c, u.s, u.d, Qd, lds, NU, NG, nt, y);
    else if constexpr (FMT == WFMT_Q4K) q4k_unit_dot<TOKC>(u.c0, u.c1, u.s, u.d, Qd, lds, NU, NG, nt, y);
    else mx_unit_dot<TOKC>(u.c, u.s, Qd, lds, NU, nt, y);
}

// A routed work unit: one item (expert, row tile) and one chunk of its tokens.
struct GvWork {
    int item0;   // item index in the grid-stride order
    int e, rt, row0, ntok, c0;
};

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
    int item0 = blockIdx.x;
    // Shared-expert items first: they are the longest, so they start at once
    // instead of trailing behind the routed ones.
    for (; item0 < total && item0 < g.tiles_s; item0 += gridDim.x) {
        const int rt = item0;
        const int ntok = a.T;
        for (int c0 = 0; c0 < ntok; c0 += g.tokc) {
            const int nt = min(g.tokc, ntok - c0);
            __syncthreads();
            if (UP) stage_plain(lds, nt, g.Ks, [xg, H = a.H, c0](int ti) { return xg + (size_t)(c0 + ti) * H; });
            else stage_plain(lds, nt, g.Ks, [shg, Fs = a.Fs, c0](int ti) { return shg + (size_t)(c0 + ti) * Fs; });
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

    // Routed items.  A wave's units form a sequence of batches (pass, matrix,
    // units ub*UB ..), two batches in flight: each batch is requested as the
    // one two places before it is reduced, the first two of a work unit
    // before its tokens are staged, and across work units.  Every batch loads
    // all UB units (indices past the row's last unit and rows past the
    // matrix's last row read that unit or row again and are not reduced), so
    // no load is conditional and the compiler's wait counts stay exact.
    constexpr int UB = gv_batch_units<FMT, TOKC>();
    constexpr int NMAT = UP ? 2 : 1;
    const int bpm = (g.UPL + UB - 1) / UB;            // batches per (pass, matrix)
    const int bpp = bpm * NMAT;                       // batches per pass
    const int nb = g.passes * bpp;
    const int nbe = nb + (nb & 1);                    // padded to whole pairs
    const int lir = lane % g.LPR, rsub = wave * (WAVE / g.LPR) + lane / g.LPR;
    const int NG = g.K / 16;
    const size_t dstr = expert_data_stride(FMT, g.rows, g.K), sstr = expert_scale_stride(FMT, g.rows, g.K);
    const int P = a.T * a.k;
    // the next routed work unit at or after item it0 (first chunk); false at the end
    auto find = [&](int it0, GvWork& w) __attribute__((always_inline)) {
        for (; it0 < total; it0 += gridDim.x) {
            const int item = it0 - g.tiles_s;
            const int e = a.active[1 + item / g.tiles];
            int row0, ntok;
            if (expert_rows(a.offsets, e, a.E, P, row0, ntok) && ntok > 0) {
                w.item0 = it0;
                w.e = e;
                w.rt = item % g.tiles;
                w.row0 = row0;
                w.ntok = ntok;
                w.c0 = 0;
                return true;
            }
        }
        return false;
    };
    // dummy: after the workgroup's last unit, every lane reads the matrix's
    // first unit (one cached line per instruction; the data is not used)
    auto issue = [&](const GvWork& w, int b, GvUnit<FMT>(&X)[UB], bool dummy) __attribute__((always_inline)) {
        b = min(b, nb - 1);
        const int ub = b % bpm, mi = (b / bpm) % NMAT, ps = b / bpp;
        const int r = min((w.rt * g.passes + ps) * g.rows_per_tile + rsub, g.rows - 1);
        const uint8_t* m = (UP && mi ? a.up : (UP ? a.gate : a.down)) + (size_t)w.e * dstr;
        const uint8_t* ms = FMT == WFMT_Q2K ? nullptr
                                            : (UP && mi ? a.up_s : (UP ? a.gate_s : a.down_s)) + (size_t)w.e * sstr;
        const int64_t f0 = dummy ? 0 : (int64_t)r * g.NU + lir;
        const int ls = dummy ? 0 : g.LPR;
#pragma unroll
        for (int i = 0; i < UB; ++i) gv_load<FMT>(X[i], m, ms, f0 + (int64_t)min(ub * UB + i, g.UPL - 1) * ls);
    };
    GvWork cur;
    if (!find(item0, cur)) return;   // uniform: no routed work for this workgroup
    GvUnit<FMT> X0[UB], X1[UB];
    issue(cur, 0, X0, false);
    issue(cur, 1, X1, false);
    for (;;) {
        const int nt = min(g.tokc, cur.ntok - cur.c0);
        // the work unit after this one: the item's next chunk, else the next item
        GvWork nxt = cur;
        bool has_next = true;
        if (cur.c0 + g.tokc < cur.ntok) nxt.c0 = cur.c0 + g.tokc;
        else has_next = find(cur.item0 + gridDim.x, nxt);
        const GvWork pf = has_next ? nxt : cur;
        __syncthreads();   // every wave is done with the previous unit's tokens
        if (UP)
            stage_routed<FMT>(lds, nt, g.K, [xg, sp = a.sorted_pair, k = a.k, H = a.H, r0 = cur.row0 + cur.c0](
                                                  int ti) { return xg + (size_t)(sp[r0 + ti] / k) * H; });
        else
            stage_routed<FMT>(lds, nt, g.K,
                                [hg, F = a.F, r0 = cur.row0 + cur.c0](int ti) { return hg + (size_t)(r0 + ti) * F; });
        __syncthreads();
        const uint8_t* xl = lds;
        float y0[TOKC], y1[TOKC];
#pragma unroll
        for (int t = 0; t < TOKC; ++t) { y0[t] = 0.0f; y1[t] = 0.0f; }
        // reduce batch b from X into the pass's sums; store the pass when it ends
        auto step = [&](int b, const GvUnit<FMT>(&X)[UB]) __attribute__((always_inline)) {
            if (b >= nb) return;
            const int ub = b % bpm, mi = (b / bpm) % NMAT, ps = b / bpp;
            const int r = (cur.rt * g.passes + ps) * g.rows_per_tile + rsub;
            const bool live = r < g.rows;
            float yb[TOKC];   // this batch's share, added to the gate or up sums below
#pragma unroll
            for (int t = 0; t < TOKC; ++t) yb[t] = 0.0f;
#pragma unroll
            for (int i = 0; i < UB; ++i) {
                const int u = ub * UB + i;
                if (live && u < g.UPL) gv_dot<FMT, TOKC>(X[i], lir + u * g.LPR, xl, g.NU, NG, nt, yb);
                if (TOKC > 1) __builtin_amdgcn_sched_barrier(0);   // one unit's LDS reads at a time
            }
#pragma unroll
            for (int t = 0; t < TOKC; ++t) {
                if (UP && mi) y1[t] += yb[t];
                else y0[t] += yb[t];
            }
            if ((b + 1) % bpp == 0) {
#pragma unroll
                for (int t = 0; t < TOKC; ++t) {
                    if (t < nt) {
                        const float v0 = group_sum(y0[t], g.LPR);
                        const float v1 = UP ? group_sum(y1[t], g.LPR) : 0.0f;
                        const size_t pr = (size_t)(cur.row0 + cur.c0 + t);
                        if (live && lir == 0) {
                            if (UP)
                                reinterpret_cast<uint16_t*>(a.h)[pr * a.F + r] = (uint16_t)f32_to_bf16(silu_f32(v0) * v1);
                            else
                                reinterpret_cast<uint16_t*>(a.expert_out)[pr * a.H + r] = (uint16_t)f32_to_bf16(v0);
                        }
                    }
                    y0[t] = 0.0f;
                    y1[t] = 0.0f;
                }
            }
        };
        for (int b = 0; b < nbe; b += 2) {
            const bool last = b + 2 >= nbe;
            step(b, X0);
            __builtin_amdgcn_sched_barrier(0);
            issue(last ? pf : cur, last ? 0 : b + 2, X0, last && !has_next);
            step(b + 1, X1);
            __builtin_amdgcn_sched_barrier(0);
            issue(last ? pf : cur, last ? 1 : b + 3, X1, last && !has_next);
        }
        if (!has_next) break;
        cur = nxt;
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
    const int P = a.T * a.k;
    const int max_active = routed ? (a.E < P ? a.E : P) : 0;
    // lanes per row: at most 8, so each lane takes more units before the
    // per-row lane reduction (down rows, K = ffn = 2048: 6-token verify step
    // 3% faster, 3-8 tokens 2-4%; Q2K gate/up rows with two-unit batches:
    // 6-token step 4% faster, 8 tokens 3-4%; 4 lanes slower).  MXFP4 and Q4K
    // gate/up rows: 8 lanes while the routed items (32 rows each) still number
    // 1536 or more (3-16 tokens 3-8% faster), else 16 (at 2 tokens, 16 routed
    // pairs, the halved item count was 2-4% slower)
    int lcap = 8;
    if (UP && FMT != WFMT_Q2K && max_active * ((g.rows + 31) / 32) < 1536) lcap = 16;
    g.LPR = gcd16(g.NU) < lcap ? gcd16(g.NU) : lcap;
    g.UPL = g.NU / g.LPR;
    g.rows_per_tile = 4 * (WAVE / g.LPR);
    // routed items of at least ~40 KB of weights: one pass of the workgroup's
    // rows for the long up rows (32 rows x 2 matrices at 8 lanes per row:
    // 150 KB of Q2K at 7168 wide), several for the short down rows (one LDS
    // staging per item)
    const double row_bytes = FMT == WFMT_Q2K ? g.K / 256.0 * 84
                             : (FMT == WFMT_Q4K ? g.K / 256.0 * 148 : g.K / 2.0 + g.K / 32.0);
    g.passes = 1;
    while (g.passes < 8 && row_bytes * g.rows_per_tile * g.passes * (UP ? 2 : 1) < 40000.0) g.passes *= 2;
    // the short down rows: twice the passes while the items still fill the
    // grid (6-token verify step 2% faster, MXFP4 and Q4K at 6 tokens 2-3%;
    // with 16 routed pairs the halved item count made 2 Q4K tokens 4% slower)
    auto tiles_of = [&](int passes) { return (g.rows + g.rows_per_tile * passes - 1) / (g.rows_per_tile * passes); };
    if (!UP && g.passes < 8 && row_bytes * g.rows_per_tile * g.passes * 2 <= 160000.0 &&
        max_active * tiles_of(2 * g.passes) >= 1024)
        g.passes *= 2;
    g.tiles = routed ? tiles_of(g.passes) : 0;
    g.Ks = UP ? a.H : a.Fs;
    g.rows_s = UP ? a.Fs : a.H;
    // shared items of 16 rows (up: row pairs), four per wave; at 7168-wide
    // rows 16-row items measured 2-4% faster steps (3-8 tokens) than one row
    // pair per wave, and 32-row items 15% slower
    g.rows_s_item = 16;
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
