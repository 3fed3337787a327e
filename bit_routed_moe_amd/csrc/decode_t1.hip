// Batch-1 decode layer (bf16 path, one token): the whole layer in two
// launches.
//
// Decode streams each touched weight byte once and is bound by memory
// bandwidth ("284B MoEを128GBノートPCに詰め込む", section
// "プリフィル790 t/sが暴く真のボトルネック").  With one token, separate route,
// permute and combine launches would cost a fifth of the step, so:
//
//   up launch    shared workgroups stage x and stream shared-expert gate+up
//                rows (a row per wave task, 64 lanes); routed workgroups rank
//                the token's router logits themselves (a block-wide rank count
//                over the E keys, no shuffles), stage x and stream routed row
//                quads (4 rows of one selected expert, 16 lanes per row); both
//                write h = silu(gate) * up as bf16.  The first routed
//                workgroup also writes the routing for the down launch;
//   down launch  each workgroup requests its first task's down rows (shared
//                and the k selected experts'), stages the k routed h rows and
//                the shared h row, and each wave task produces rows of y: the
//                shared down rows plus the experts' down rows weighted by the
//                router weights, summed in slot order in fp32 and rounded once
//                to bf16.  There is no expert_out round trip and no separate
//                combine.
//
// Tasks go to waves with a stride of the grid's wave count (down: an equal
// contiguous block per workgroup).  For the 7168/2048/256-expert top-8 layer
// with a 2048-row shared expert, each CU runs one shared and one routed
// workgroup (two shared rows per shared wave, four routed quads per routed
// wave: 530 KB of weights) and 14 down tasks (265 KB), so every CU streams
// the same bytes.  A wave keeps the next task half's rows in
// flight while it reduces the current one.
//
// Weight decode and the dot products are those of the GEMV kernels (vecdot.hpp):
// Q2K codes are reduced against pre-scaled activations without forming weight
// values, MXFP4 bytes convert exactly to bf16 pairs, bf16 rows are dotted as is.
#include "formats.hpp"
#include "launch.hpp"
#include "vecdot.hpp"

namespace ds4 {

namespace {

constexpr int T1_KMAX = 16;
constexpr int T1_UP_THREADS = 256;

struct T1Args {
    int H, F, Fs, E, k;
    const float* logits;    // [E]
    const uint16_t* x;      // [H] bf16
    const uint8_t *gate, *up, *down, *gate_s, *up_s, *down_s;
    const uint16_t *sh_gate, *sh_up, *sh_down;
    uint16_t* h;            // [k][F] bf16, slot order
    uint16_t* sh_h;         // [Fs] bf16
    uint16_t* y;            // [H] bf16
    int32_t* sel;           // [k] the routing, written by the up launch for the down launch
    float* selw;            // [k]
};

// Top-k of one token's logits by rank counting: expert e is kept at slot
// rank(e) = #{i : key_i > key_e} when that is below k, under the router's key
// (logit descending, lower index first on ties, -0 == +0).  Weights are the
// softmax over the kept logits, summed in slot order.  Block-wide, over the
// keys already in LDS (written before a barrier); ends with the results in
// LDS and a barrier.
__device__ void t1_rank(int E, int k, const uint64_t* keys, int* sel, float* selw) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const uint64_t me = keys[e];
        int rank = 0;
        for (int i = 0; i < E; ++i) rank += keys[i] > me ? 1 : 0;
        if (rank < k) {
            sel[rank] = e;
            selw[rank] = key_value(me);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const float l0 = selw[0];
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) {
            const float ex = expf(selw[j] - l0);
            selw[j] = ex;
            sum += ex;
        }
        for (int j = 0; j < k; ++j) selw[j] = selw[j] / sum;
    }
    __syncthreads();
}

// Router logits of this thread (up to T1_LPT per thread, E <= T1_LPT * blockDim).
constexpr int T1_LPT = 4;
__device__ __forceinline__ void t1_load_logits(const float* __restrict__ logits, int E, float* lg) {
#pragma unroll
    for (int m = 0; m < T1_LPT; ++m) {
        const int e = threadIdx.x + m * blockDim.x;
        if (e < E) lg[m] = logits[e];
    }
}
__device__ __forceinline__ void t1_store_keys(const float* lg, int E, uint64_t* keys) {
#pragma unroll
    for (int m = 0; m < T1_LPT; ++m) {
        const int e = threadIdx.x + m * blockDim.x;
        if (e < E) keys[e] = route_key(lg[m], e);
    }
}

// ---- per-lane dot products over a task half's loaded bytes ------------------------
// Staged activations of one Q2K unit (64 weights): 8 bf16-pair pieces, the 4
// groups' -C and S.
struct T1XQ {
    u32x4 p[8];
    f32x4 c, s;
};

__device__ __forceinline__ void t1_load_xq(T1XQ& x, const u32x4* __restrict__ xq, const float* __restrict__ C,
                                           const float* __restrict__ S, int NQ, int Q) {
#pragma unroll
    for (int v = 0; v < 8; ++v) x.p[v] = xq[v * NQ + Q];
    x.c = *reinterpret_cast<const f32x4*>(C + 4 * Q);
    x.s = *reinterpret_cast<const f32x4*>(S + 4 * Q);
}

template <int Q4>
__device__ __forceinline__ void t1_q2k_group(uint32_t cw, const T1XQ& x, uint32_t sn, uint32_t mn, float& P,
                                             float& M) {
    uint32_t e[8];
    q2k_expand(cw, e);
    float acc = x.c[Q4];
    acc = dot2bf(e[0], x.p[2 * Q4][0], acc);
    acc = dot2bf(e[1], x.p[2 * Q4][1], acc);
    acc = dot2bf(e[2], x.p[2 * Q4][2], acc);
    acc = dot2bf(e[3], x.p[2 * Q4][3], acc);
    acc = dot2bf(e[4], x.p[2 * Q4 + 1][0], acc);
    acc = dot2bf(e[5], x.p[2 * Q4 + 1][1], acc);
    acc = dot2bf(e[6], x.p[2 * Q4 + 1][2], acc);
    acc = dot2bf(e[7], x.p[2 * Q4 + 1][3], acc);
    P = fmaf(ubyte_f32<Q4>(sn), acc, P);
    M = fmaf(ubyte_f32<Q4>(mn), x.s[Q4], M);
}

// This lane's share of a Q2K row: NU units (quads Q = lir + QS*u).  One
// unit's staged activations and products at a time: the other wave on the
// SIMD covers the LDS latency.
template <int NU, int QS = 16>
__device__ __forceinline__ float t1_q2k_dot(const u32x4* c, const uint32_t* s, const uint32_t* d, int lir,
                                            const u32x4* __restrict__ xq, const float* __restrict__ C,
                                            const float* __restrict__ S, int NQ) {
    float y = 0.0f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int Q = lir + QS * u;
        T1XQ x;
        // groups 0, 1 of the unit, then 2, 3: half the staged activations
        // live at a time (register pressure)
#pragma unroll
        for (int v = 0; v < 4; ++v) x.p[v] = xq[v * NQ + Q];
        x.c = *reinterpret_cast<const f32x4*>(C + 4 * Q);
        x.s = *reinterpret_cast<const f32x4*>(S + 4 * Q);
        const float dd = half_bits_to_f32(d[u] & 0xFFFFu);
        const float dm = half_bits_to_f32(d[u] >> 16);
        const uint32_t sn = s[u] & 0x0F0F0F0Fu, mn = (s[u] >> 4) & 0x0F0F0F0Fu;
        float P = 0.0f, M = 0.0f;
        t1_q2k_group<0>(c[u][0], x, sn, mn, P, M);
        t1_q2k_group<1>(c[u][1], x, sn, mn, P, M);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 4; v < 8; ++v) x.p[v] = xq[v * NQ + Q];
        t1_q2k_group<2>(c[u][2], x, sn, mn, P, M);
        t1_q2k_group<3>(c[u][3], x, sn, mn, P, M);
        y = fmaf(dd, P, y);
        y = fmaf(-dm, M, y);
        __builtin_amdgcn_sched_barrier(0);   // one unit at a time (register pressure)
    }
    return y;
}

// This lane's share of a Q4K row: NU units of 64 weights (two code pieces
// each, quads Q = lir + QS*u), against activations staged by
// stage_q4k_group (pairs (x_n, x_{n+4}), and the group sums S), one group's
// two staged pieces at a time.
template <int NU, int QS = 16>
__device__ __forceinline__ float t1_q4k_dot(const u32x4* c, const uint32_t* s, const uint32_t* d, int lir,
                                            const u32x4* __restrict__ xq, const float* __restrict__ S, int NQ) {
    float y = 0.0f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int Q = lir + QS * u;
        const uint32_t sn = s[u] & 0x0F0F0F0Fu, mn = (s[u] >> 4) & 0x0F0F0F0Fu;
        float P = 0.0f, M = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 xa = xq[(2 * q) * NQ + Q];
            const u32x4 xb = xq[(2 * q + 1) * NQ + Q];
            const float sg = S[4 * Q + q];
            uint32_t e[4];
            float acc = -128.0f * sg;
            q4k_expand(c[2 * u + (q >> 1)][2 * (q & 1)], e);
            acc = dot2bf(e[0], xa[0], acc);
            acc = dot2bf(e[1], xa[1], acc);
            acc = dot2bf(e[2], xa[2], acc);
            acc = dot2bf(e[3], xa[3], acc);
            q4k_expand(c[2 * u + (q >> 1)][2 * (q & 1) + 1], e);
            acc = dot2bf(e[0], xb[0], acc);
            acc = dot2bf(e[1], xb[1], acc);
            acc = dot2bf(e[2], xb[2], acc);
            acc = dot2bf(e[3], xb[3], acc);
            const float sq = q == 0 ? ubyte_f32<0>(sn) : q == 1 ? ubyte_f32<1>(sn) : q == 2 ? ubyte_f32<2>(sn)
                                                                                             : ubyte_f32<3>(sn);
            const float mq = q == 0 ? ubyte_f32<0>(mn) : q == 1 ? ubyte_f32<1>(mn) : q == 2 ? ubyte_f32<2>(mn)
                                                                                             : ubyte_f32<3>(mn);
            P = fmaf(sq, acc, P);
            M = fmaf(mq, sg, M);
        }
        y = fmaf(half_bits_to_f32(d[u] & 0xFFFFu), P, y);
        y = fmaf(-half_bits_to_f32(d[u] >> 16), M, y);
        __builtin_amdgcn_sched_barrier(0);   // one unit at a time (register pressure)
    }
    return y;
}

template <int NB, int QS = 16>
__device__ __forceinline__ float t1_mx_dot(const u32x4* c, const uint32_t* s, int lir, const u32x4* __restrict__ xm,
                                           int NBR) {
    float y = 0.0f;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int B = lir + QS * u;
        float acc = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const u32x4 xa = xm[v * NBR + B];
            acc = dot2bf(fp4x2_to_bf16x2<0>(c[u][v]), xa[0], acc);
            acc = dot2bf(fp4x2_to_bf16x2<1>(c[u][v]), xa[1], acc);
            acc = dot2bf(fp4x2_to_bf16x2<2>(c[u][v]), xa[2], acc);
            acc = dot2bf(fp4x2_to_bf16x2<3>(c[u][v]), xa[3], acc);
        }
        y += ldexpf(acc, (int)(s[u] & 0xFFu) - 127);
        __builtin_amdgcn_sched_barrier(0);
    }
    return y;
}

template <int NC>
__device__ __forceinline__ float t1_bf16_dot(const u32x4* c, const u32x4* __restrict__ xs, int c0, int cstride) {
    float y = 0.0f;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
        const u32x4 xv = xs[c0 + cstride * u];
        y = dot2bf(c[u][0], xv[0], y);
        y = dot2bf(c[u][1], xv[1], y);
        y = dot2bf(c[u][2], xv[2], y);
        y = dot2bf(c[u][3], xv[3], y);
    }
    return y;
}

// ---- up launch -----------------------------------------------------------------
// Workgroups [0, gs) take shared rows, the rest routed row quads.  With two
// workgroups per CU, a CU runs one of each, so every SIMD interleaves a
// shared wave (bf16 rows, light on VALU) with a routed wave (2-bit or 4-bit
// rows, heavy on VALU).  Each wave keeps the next task's rows in flight while
// it reduces the current one.  The loops hold no conditional load: the wait
// counts the compiler derives are exact, so a wave waits only for the rows it
// is about to reduce.
// HC = H / 512: 16-byte chunks per lane of a shared row (64 lanes), MXFP4 blocks
// per lane of a routed row (16 lanes), twice the Q2K units per lane.
template <int HC>
struct T1ShBuf {
    u32x4 c[HC];
};
template <int FMT, int HC>
struct T1RtBuf {
    u32x4 c[FMT == WFMT_Q2K ? HC / 2 : HC];
    uint32_t s[FMT == WFMT_MX ? HC : HC / 2];
    uint32_t d[FMT == WFMT_MX ? 1 : HC / 2];
};

// LDS: shared workgroups xs [H/8] (x in natural chunks); routed workgroups
// xr (Q2K xq [8][H/64] + C [H/16] + S [H/16]; MXFP4 xm [4][H/32]), keys [E],
// sel, selw.
// Bytes of the routed activation staging beyond the H bf16 pieces: Q2K the
// group constants C and sums S, Q4K the sums S.
__host__ __device__ inline size_t t1_xs_extra(int FMT, int K) {
    return FMT == WFMT_Q2K ? (size_t)K / 16 * 8 : (FMT == WFMT_Q4K ? (size_t)K / 16 * 4 : 0);
}

size_t t1_up_lds_bytes(int FMT, int H, int E) {
    const size_t rt = (size_t)H * 2 + t1_xs_extra(FMT, H) + (size_t)E * 8 + T1_KMAX * 8;
    const size_t sh = (size_t)H * 2;
    return rt > sh ? rt : sh;
}

template <int HC>
__device__ __forceinline__ void t1_sh_issue(const uint16_t* __restrict__ w, int row, int lane, T1ShBuf<HC>& b) {
    const u32x4* p = reinterpret_cast<const u32x4*>(w + (size_t)row * HC * 512);
#pragma unroll
    for (int u = 0; u < HC; ++u) b.c[u] = p[lane + 64 * u];
}

template <int FMT, int HC>
__device__ __forceinline__ void t1_rt_issue(const T1Args& a, const uint8_t* m, const uint8_t* ms, int r, int lir,
                                            T1RtBuf<FMT, HC>& b) {
    const int H = HC * 512;
    if (FMT == WFMT_Q4K) {
        const u32x4* row = reinterpret_cast<const u32x4*>(m + (size_t)r * (H / 2));
        const uint8_t* recs = ms + (size_t)r * (H / 256) * Q4K_PARAM_BYTES;
#pragma unroll
        for (int u = 0; u < HC / 2; ++u) {
            const int Q = lir + 16 * u;
            b.c[2 * u] = row[2 * Q];
            b.c[2 * u + 1] = row[2 * Q + 1];
            const uint8_t* rec = recs + (Q >> 2) * Q4K_PARAM_BYTES;
            b.s[u] = ld_u32(rec + 4 * (Q & 3));
            b.d[u] = ld_u32(rec + 16);
        }
    } else if (FMT == 1) {
        const uint8_t* blk = m + ((size_t)r * (H / 256) + (lir >> 2)) * Q2K_BLOCK_BYTES;
        const int jq = lir & 3;
#pragma unroll
        for (int u = 0; u < HC / 2; ++u) {
            const uint8_t* bu = blk + 4 * Q2K_BLOCK_BYTES * u;
            b.c[u] = *reinterpret_cast<const u32x4*>(bu + 16 + 16 * jq);
            b.s[u] = ld_u32(bu + 4 * jq);
            b.d[u] = ld_u32(bu + 80);
        }
    } else {
        const uint8_t* row = m + (size_t)r * (H / 2);
        const uint8_t* sc = ms + (size_t)r * (H / 32);
#pragma unroll
        for (int u = 0; u < HC; ++u) {
            b.c[u] = *reinterpret_cast<const u32x4*>(row + 16 * (lir + 16 * u));
            b.s[u] = sc[lir + 16 * u];
        }
    }
}

template <int FMT, int HC>
__device__ __forceinline__ float t1_rt_reduce(const uint8_t* lds, int lir, const T1RtBuf<FMT, HC>& b) {
    const int H = HC * 512;
    const u32x4* xr = reinterpret_cast<const u32x4*>(lds);
    float v;
    if (FMT == WFMT_Q4K) {
        // one unit at a time: the whole row's expansions would not fit the registers
        v = 0.0f;
#pragma unroll
        for (int u = 0; u < HC / 2; ++u) {
            q4k_unit_dot<1>(b.c[2 * u], b.c[2 * u + 1], b.s[u], b.d[u], lir + 16 * u, lds, H / 64, H / 16, 1, &v);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if (FMT == 1) {
        const float* C = reinterpret_cast<const float*>(xr + H / 8);
        v = t1_q2k_dot<HC / 2>(b.c, b.s, b.d, lir, xr, C, C + H / 16, H / 64);
    } else {
        v = t1_mx_dot<HC>(b.c, b.s, lir, xr, H / 32);
    }
    return group_sum(v, 16);
}

template <int FMT, int HC>
__global__ __launch_bounds__(T1_UP_THREADS, 2) void t1_up_kernel(T1Args a, int gs) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int H = HC * 512;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wpb = T1_UP_THREADS / 64;
    if ((int)blockIdx.x < gs) {
        // shared rows: x in natural chunks, then gate/up rows
        constexpr int XPT = (HC * 64 + T1_UP_THREADS - 1) / T1_UP_THREADS;   // x chunks per thread
        const int n = a.Fs, NW = gs * wpb;
        int t = blockIdx.x * wpb + wave;
        const u32x4* xg = reinterpret_cast<const u32x4*>(a.x);
        u32x4 xc[XPT];
#pragma unroll
        for (int m = 0; m < XPT; ++m) xc[m] = xg[min((int)threadIdx.x + m * T1_UP_THREADS, HC * 64 - 1)];
        T1ShBuf<HC> G, U;
        const int t0 = min(t, n - 1);
        t1_sh_issue<HC>(a.sh_gate, t0, lane, G);
        t1_sh_issue<HC>(a.sh_up, t0, lane, U);
        u32x4* xs = reinterpret_cast<u32x4*>(lds);
#pragma unroll
        for (int m = 0; m < XPT; ++m) {
            const int c = threadIdx.x + m * T1_UP_THREADS;
            if (c < HC * 64) xs[c] = xc[m];
        }
        __syncthreads();
        if (t >= n) return;
        // the next row is requested as each buffer is reduced; past the
        // wave's last row the request reads x itself (one row of H bf16, in
        // cache), so no load is conditional
        for (;;) {
            const int tn = t + NW;
            const bool live = tn < n;
            const float g = wave_sum(t1_bf16_dot<HC>(G.c, xs, lane, 64));
            __builtin_amdgcn_sched_barrier(0);
            t1_sh_issue<HC>(live ? a.sh_gate : a.x, live ? tn : 0, lane, G);
            const float u = wave_sum(t1_bf16_dot<HC>(U.c, xs, lane, 64));
            __builtin_amdgcn_sched_barrier(0);
            t1_sh_issue<HC>(live ? a.sh_up : a.x, live ? tn : 0, lane, U);
            if (lane == 0) a.sh_h[t] = (uint16_t)f32_to_bf16(silu_f32(g) * u);
            if (tn >= n) break;
            t = tn;
        }
        return;
    }

    // routed row quads: routing, x in the routed layout, then gate/up quads
    uint8_t* xr = lds;
    const size_t xr_bytes = (size_t)H * 2 + t1_xs_extra(FMT, H);
    uint64_t* keys = reinterpret_cast<uint64_t*>(lds + xr_bytes);
    int* sel = reinterpret_cast<int*>(keys + a.E);
    float* selw = reinterpret_cast<float*>(sel + T1_KMAX);
    constexpr int GPT = (HC * 32 + T1_UP_THREADS - 1) / T1_UP_THREADS;   // x groups of 16 per thread
    float lg[T1_LPT];
#pragma unroll
    for (int m = 0; m < T1_LPT; ++m) lg[m] = a.logits[min((int)threadIdx.x + m * T1_UP_THREADS, a.E - 1)];
    const u32x4* xg = reinterpret_cast<const u32x4*>(a.x);
    u32x4 xl[GPT][2];
#pragma unroll
    for (int m = 0; m < GPT; ++m) {
        const int Gi = min((int)threadIdx.x + m * T1_UP_THREADS, HC * 32 - 1);
        xl[m][0] = xg[2 * Gi];
        xl[m][1] = xg[2 * Gi + 1];
    }
    t1_store_keys(lg, a.E, keys);
#pragma unroll
    for (int m = 0; m < GPT; ++m) {
        const int Gi = threadIdx.x + m * T1_UP_THREADS;
        if (Gi < HC * 32) {
            if (FMT == WFMT_Q2K) stage_q2k_group(xr, 1, H, 0, Gi, xl[m][0], xl[m][1]);
            else if (FMT == WFMT_Q4K) stage_q4k_group(xr, 1, H, 0, Gi, xl[m][0], xl[m][1]);
            else stage_mx_group(xr, 1, H, 0, Gi, xl[m][0], xl[m][1]);
        }
    }
    __syncthreads();
    t1_rank(a.E, a.k, keys, sel, selw);   // ends with a barrier
    if ((int)blockIdx.x == gs && (int)threadIdx.x < a.k) {   // the routing, for the down launch
        a.sel[threadIdx.x] = sel[threadIdx.x];
        a.selw[threadIdx.x] = selw[threadIdx.x];
    }

    const int n = a.k * (a.F >> 2), quads = a.F >> 2;
    const int NW = (gridDim.x - gs) * wpb;
    const int t0 = (blockIdx.x - gs) * wpb + wave;
    if (t0 >= n) return;
    const int lir = lane & 15, rq = lane >> 4;
    const size_t dstr = expert_data_stride(FMT, a.F, H), sstr = expert_scale_stride(FMT, a.F, H);
    const int tlast = t0 + (n - 1 - t0) / NW * NW;   // this wave's last task
    // Row half i of this wave: gate (i even) or up (i odd) rows of task
    // t0 + (i / 2) * NW.  Halves past the wave's last task read the first
    // bytes of x instead (row 0 of a matrix at x: every offset a row half
    // reads is below the 2*H bytes of x, which the workgroup has just read,
    // so they hit the cache); no load is conditional, so the compiler's wait
    // counts stay exact.
    const uint8_t* const xb = reinterpret_cast<const uint8_t*>(a.x);
    auto issue = [&](int i, T1RtBuf<FMT, HC>& B) {
        const int tt = t0 + (i >> 1) * NW;
        const bool live = tt <= tlast;
        const int tc = live ? tt : tlast;
        const int j = tc / quads;
        const size_t e = (size_t)sel[j];
        const int r = live ? 4 * (tc - j * quads) + rq : 0;
        const uint8_t* m = live ? ((i & 1) ? a.up : a.gate) + e * dstr : xb;
        const uint8_t* ms = FMT != WFMT_Q2K ? (live ? ((i & 1) ? a.up_s : a.gate_s) + e * sstr : xb) : nullptr;
        t1_rt_issue<FMT, HC>(a, m, ms, r, lir, B);
    };
    auto store = [&](int tt, float g, float u) {
        if (lir == 0) {
            const int j = tt / quads;
            a.h[(size_t)j * a.F + 4 * (tt - j * quads) + rq] = (uint16_t)f32_to_bf16(silu_f32(g) * u);
        }
    };
    // Two buffers, the gate and up halves of a task; each half of the next
    // task is requested as soon as its buffer is reduced.
    T1RtBuf<FMT, HC> G, U;
    issue(0, G);
    issue(1, U);
    for (int i = 0;; i += 2) {
        const int ta = t0 + (i >> 1) * NW;
        const float g = t1_rt_reduce<FMT, HC>(xr, lir, G);
        __builtin_amdgcn_sched_barrier(0);
        issue(i + 2, G);
        const float u = t1_rt_reduce<FMT, HC>(xr, lir, U);
        __builtin_amdgcn_sched_barrier(0);
        issue(i + 3, U);
        store(ta, g, u);
        if (ta + NW >= n) break;
    }
}

// ---- down launch ---------------------------------------------------------------
// NU: Q2K units (64 weights) or MXFP4 blocks per lane of a routed down row
// (F / 1024 or F / 512, 16 lanes per row); D: expert slots in flight.
template <int FMT, int NU>
struct T1DnBuf {
    u32x4 c[FMT == WFMT_Q4K ? 2 * NU : NU];
    uint32_t s[NU];
    uint32_t d[FMT == WFMT_MX ? 1 : NU];
};


struct T1DnLds {
    u32x4* hr;      // routed h: Q2K hq [k][8][F/64] + C [k][F/16] + S [k][F/16]; Q4K hq [k][8][F/64] +
                    // S [k][F/16]; MXFP4 hm [k][4][F/32]
    const float *C, *S;
    u32x4* hs;      // shared h, natural chunks [Fs/8]
};

__device__ __forceinline__ T1DnLds t1_dn_lds(uint8_t* lds, int FMT, int F, int Fs, int E, int k) {
    T1DnLds L;
    L.hr = reinterpret_cast<u32x4*>(lds);
    L.C = reinterpret_cast<const float*>(L.hr + (size_t)k * F / 8);
    L.S = FMT == WFMT_Q4K ? L.C : L.C + (size_t)k * F / 16;
    L.hs = reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(L.hr + (size_t)k * F / 8) + t1_xs_extra(FMT, k * F));
    (void)Fs;
    (void)E;
    return L;
}

size_t t1_dn_lds_bytes(int FMT, int F, int Fs, int E, int k) {
    (void)E;
    return (size_t)k * F * 2 + t1_xs_extra(FMT, k * F) + (size_t)Fs * 2;
}

template <int FMT, int NU, int LPR>
__device__ __forceinline__ void t1_dn_issue(const T1Args& a, int e, int r, int lir, T1DnBuf<FMT, NU>& b) {
    if (FMT == WFMT_Q4K) {
        const u32x4* row = reinterpret_cast<const u32x4*>(a.down + (size_t)e * expert_data_stride(WFMT_Q4K, a.H, a.F) +
                                                          (size_t)r * (a.F / 2));
        const uint8_t* recs = a.down_s + (size_t)e * expert_scale_stride(WFMT_Q4K, a.H, a.F) +
                              (size_t)r * (a.F / 256) * Q4K_PARAM_BYTES;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int Q = lir + LPR * u;
            b.c[2 * u] = row[2 * Q];
            b.c[2 * u + 1] = row[2 * Q + 1];
            const uint8_t* rec = recs + (Q >> 2) * Q4K_PARAM_BYTES;
            b.s[u] = ld_u32(rec + 4 * (Q & 3));
            b.d[u] = ld_u32(rec + 16);
        }
    } else if (FMT == 1) {
        const uint8_t* m = a.down + (size_t)e * expert_data_stride(1, a.H, a.F);
        const uint8_t* blk = m + ((size_t)r * (a.F / 256) + (lir >> 2)) * Q2K_BLOCK_BYTES;
        const int jq = lir & 3;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const uint8_t* bu = blk + (LPR / 4) * Q2K_BLOCK_BYTES * u;
            b.c[u] = *reinterpret_cast<const u32x4*>(bu + 16 + 16 * jq);
            b.s[u] = ld_u32(bu + 4 * jq);
            b.d[u] = ld_u32(bu + 80);
        }
    } else {
        const uint8_t* m = a.down + (size_t)e * expert_data_stride(2, a.H, a.F) + (size_t)r * (a.F / 2);
        const uint8_t* sc = a.down_s + (size_t)e * expert_scale_stride(2, a.H, a.F) + (size_t)r * (a.F / 32);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            b.c[u] = *reinterpret_cast<const u32x4*>(m + 16 * (lir + LPR * u));
            b.s[u] = sc[lir + LPR * u];
        }
    }
}

// LPR lanes per down row (RPW = 64 / LPR rows per wave task), NU units or
// blocks per lane per expert row, D expert slots in flight.  KT: the exact
// top-k when it is a compile-time constant (slot loops unrolled without
// guards, so the compiler's wait counts are exact), 0 for any k <= T1_KMAX.
// NSC: shared-row chunks per lane when constant, -1 for any Fs.
template <int FMT, int NU, int LPR, int D, int KT, int NSC>
__global__ __launch_bounds__(512, 2) void t1_down_kernel(T1Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int RPW = 64 / LPR;
    constexpr int SCM = 2048 / 8 / LPR;   // shared chunks per lane at most (Fs <= 2048)
    const int F = FMT == WFMT_MX ? NU * 32 * LPR : NU * 64 * LPR;
    const int KM = KT > 0 ? KT : T1_KMAX;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lir = lane % LPR, rsub = lane / LPR;
    const int wpb = blockDim.x >> 6;
    const T1DnLds L = t1_dn_lds(lds, FMT, F, a.Fs, a.E, a.k);
    const int k = KT > 0 ? KT : a.k;
    const int n = a.H / RPW;
    const int bd = blockDim.x;   // >= 256
    // tasks: a contiguous block per workgroup (every CU the same count),
    // strided over its waves
    const int tpb = (n + gridDim.x - 1) / gridDim.x;
    const int tend = min(n, (int)(blockIdx.x + 1) * tpb);
    const int nsc = a.Fs / (8 * LPR);   // shared chunks per lane
    // The routing comes from the up launch.  The first task's rows (shared and
    // routed) are requested before anything else, then h is loaded and
    // staged: waiting for h then also waits for those rows, which the task
    // needs next anyway.
    int sel[KM];
    float selw[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        if (j < k) {
            sel[j] = a.sel[j];
            selw[j] = a.selw[j];
        }
    }
    int t = blockIdx.x * tpb + wave;
    const uint16_t* shw = a.Fs > 0 ? a.sh_down : a.h;
    u32x4 sc[NSC >= 0 ? NSC : SCM];
    const int nsc_l = NSC >= 0 ? NSC : nsc;
    auto load_sc = [&](int tt) {
        const u32x4* sw = reinterpret_cast<const u32x4*>(shw + (size_t)(RPW * tt + rsub) * a.Fs);
#pragma unroll
        for (int u = 0; u < (NSC >= 0 ? NSC : SCM); ++u)
            if (NSC >= 0 || u < nsc_l) sc[u] = sw[lir + LPR * u];
    };
    T1DnBuf<FMT, NU> R[D];
    auto issue_first = [&](int tt) {
        const int r = RPW * tt + rsub;
        load_sc(tt);
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (j < k) t1_dn_issue<FMT, NU, LPR>(a, sel[j], r, lir, R[j]);
    };
    if (t < tend) issue_first(t);
    const int NG = F / 16, NI = k * NG;
    {
        // two groups per thread loaded together, then any remainder
        u32x4 hl[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = min((int)threadIdx.x + m * bd, NI - 1);
            const u32x4* src = reinterpret_cast<const u32x4*>(a.h + (size_t)(i / NG) * F) + 2 * (i % NG);
            hl[m][0] = src[0];
            hl[m][1] = src[1];
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = threadIdx.x + m * bd;
            if (i < NI) {
                if (FMT == WFMT_Q2K)
                    stage_q2k_group(reinterpret_cast<uint8_t*>(L.hr), k, F, i / NG, i % NG, hl[m][0], hl[m][1]);
                else if (FMT == WFMT_Q4K)
                    stage_q4k_group(reinterpret_cast<uint8_t*>(L.hr), k, F, i / NG, i % NG, hl[m][0], hl[m][1]);
                else stage_mx_group(reinterpret_cast<uint8_t*>(L.hr), k, F, i / NG, i % NG, hl[m][0], hl[m][1]);
            }
        }
    }
    for (int i = threadIdx.x + 2 * bd; i < NI; i += bd) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.h + (size_t)(i / NG) * F) + 2 * (i % NG);
        const u32x4 lo = src[0], hi = src[1];
        if (FMT == WFMT_Q2K) stage_q2k_group(reinterpret_cast<uint8_t*>(L.hr), k, F, i / NG, i % NG, lo, hi);
        else if (FMT == WFMT_Q4K) stage_q4k_group(reinterpret_cast<uint8_t*>(L.hr), k, F, i / NG, i % NG, lo, hi);
        else stage_mx_group(reinterpret_cast<uint8_t*>(L.hr), k, F, i / NG, i % NG, lo, hi);
    }
    for (int i = threadIdx.x; i < a.Fs / 8; i += bd) L.hs[i] = reinterpret_cast<const u32x4*>(a.sh_h)[i];
    __syncthreads();
    if (t >= tend) return;

    bool first = true;
    for (;;) {
        const int r = RPW * t + rsub;
        if (!first) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                if (j < k) t1_dn_issue<FMT, NU, LPR>(a, sel[j], r, lir, R[j]);
        }
        first = false;
        float s = 0.0f;
#pragma unroll
        for (int u = 0; u < (NSC >= 0 ? NSC : SCM); ++u) {
            if (NSC >= 0 || u < nsc_l) {
                const u32x4 xv = L.hs[lir + LPR * u];
                s = dot2bf(sc[u][0], xv[0], s);
                s = dot2bf(sc[u][1], xv[1], s);
                s = dot2bf(sc[u][2], xv[2], s);
                s = dot2bf(sc[u][3], xv[3], s);
            }
            if ((u & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // 4 chunks' LDS reads at a time
        }
        s = group_sum(s, LPR);
        const int tn = t + wpb;
        if (tn < tend) load_sc(tn);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            if (j < k) {
                T1DnBuf<FMT, NU>& b = R[j % D];
                float v;
                if (FMT == WFMT_Q4K)
                    v = t1_q4k_dot<NU, LPR>(b.c, b.s, b.d, lir, L.hr + (size_t)j * F / 8, L.S + (size_t)j * F / 16,
                                            F / 64);
                else if (FMT == 1)
                    v = t1_q2k_dot<NU, LPR>(b.c, b.s, b.d, lir, L.hr + (size_t)j * F / 8, L.C + (size_t)j * F / 16,
                                            L.S + (size_t)j * F / 16, F / 64);
                else
                    v = t1_mx_dot<NU, LPR>(b.c, b.s, lir, L.hr + (size_t)j * F / 8, F / 32);
                if (j + D < k) t1_dn_issue<FMT, NU, LPR>(a, sel[j + D], r, lir, b);
                acc = fmaf(selw[j], group_sum(v, LPR), acc);
                // keep each slot's LDS reads with its own products: hoisting
                // them all would exhaust the registers
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (lir == 0) a.y[r] = (uint16_t)f32_to_bf16(acc + s);
        if (tn >= tend) break;
        t = tn;
    }
}

template <int FMT, int HC>
hipError_t t1_launch_up(const T1Args& a, int gs, int grid, size_t lds, hipStream_t s) {
    return launch_stage(STAGE_FFN_UP, t1_up_kernel<FMT, HC>, dim3(grid), dim3(T1_UP_THREADS), lds, s, a, gs);
}

template <int FMT, int NU, int LPR, int D>
hipError_t t1_launch_dn(const T1Args& a, int grid, int threads, size_t lds, hipStream_t s) {
    if (a.k == 8 && a.Fs == 2048)
        return launch_stage(STAGE_FFN_DOWN, t1_down_kernel<FMT, NU, LPR, D, 8, 2048 / 8 / LPR>, dim3(grid),
                            dim3(threads), lds, s, a);
    return launch_stage(STAGE_FFN_DOWN, t1_down_kernel<FMT, NU, LPR, D, 0, -1>, dim3(grid), dim3(threads), lds, s,
                        a);
}

}  // namespace

bool t1_supported(int wfmt, int H, int F, int Fs, int E, int k) {
    if (wfmt != WFMT_Q2K && wfmt != WFMT_MX && wfmt != WFMT_Q4K) return false;
    // Q4K rows carry twice the code registers of Q2K: the two-launch kernels
    // hold them without scratch spills up to 7168-wide rows (the up launch's
    // two buffers of 7 units per lane) with ffn 2048; other Q4K shapes take
    // the GEMV launches.
    if (wfmt == WFMT_Q4K && (H > 7168 || F != 2048)) return false;
    if (H != 1024 && H != 2048 && H != 4096 && H != 7168 && H != 8192) return false;
    if (F != 1024 && F != 2048) return false;
    if (Fs < 0 || Fs % 256 != 0 || Fs > 2048) return false;
    if (k < 1 || k > T1_KMAX || E < k || E > 1024) return false;
    return t1_up_lds_bytes(wfmt, H, E) <= 65536 && t1_dn_lds_bytes(wfmt, F, Fs, E, k) <= 65536;
}

hipError_t launch_layer_t1(const T1Params& p, hipStream_t s) {
    T1Args a;
    a.H = p.H;
    a.F = p.F;
    a.Fs = p.Fs;
    a.E = p.E;
    a.k = p.k;
    a.logits = p.logits;
    a.x = p.x;
    a.gate = p.gate;
    a.up = p.up;
    a.down = p.down;
    a.gate_s = p.gate_s;
    a.up_s = p.up_s;
    a.down_s = p.down_s;
    a.sh_gate = p.sh_gate;
    a.sh_up = p.sh_up;
    a.sh_down = p.sh_down;
    a.h = p.h;
    a.sh_h = p.sh_h;
    a.y = p.y;
    a.sel = p.sel;
    a.selw = p.selw;
    if (!t1_supported(p.wfmt, a.H, a.F, a.Fs, a.E, a.k)) return hipErrorInvalidValue;

    // up: shared workgroups then routed workgroups, at most 512 in all (two
    // per CU); each CU runs one of each when both kinds fill 256
    const int wpb_up = T1_UP_THREADS / 64;
    const int n_rt = a.k * (a.F / 4);
    int gs = a.Fs > 0 ? (a.Fs + wpb_up - 1) / wpb_up : 0;
    if (gs > 256) gs = 256;
    int gr = (n_rt + wpb_up - 1) / wpb_up;
    if (gr > 512 - gs) gr = 512 - gs;
    const size_t lu = t1_up_lds_bytes(p.wfmt, a.H, a.E);
    hipError_t e;
    const int HC = a.H / 512;
#define T1_UP(F_, HC_) \
    if (p.wfmt == F_ && HC == HC_) e = t1_launch_up<F_, HC_>(a, gs, gs + gr, lu, s);
    e = hipErrorInvalidValue;
    T1_UP(1, 2) T1_UP(1, 4) T1_UP(1, 8) T1_UP(1, 14) T1_UP(1, 16)
    T1_UP(2, 2) T1_UP(2, 4) T1_UP(2, 8) T1_UP(2, 14) T1_UP(2, 16)
    T1_UP(4, 2) T1_UP(4, 4) T1_UP(4, 8) T1_UP(4, 14)
#undef T1_UP
    if (e != hipSuccess) return e;

    // down: row tasks in equal contiguous blocks over 256 workgroups (one per
    // CU) of 8 waves (two per SIMD); 16 lanes per row for F = 1024, 32 for
    // F = 2048, so a lane holds one Q2K unit (two MXFP4 blocks) per expert row
    const int lpr = a.F == 1024 ? 16 : 32;
    const int n_dn = a.H / (64 / lpr);
    const int grid_dn = n_dn < 256 ? n_dn : 256;
    const size_t ld = t1_dn_lds_bytes(p.wfmt, a.F, a.Fs, a.E, a.k);
#define T1_DN(F_, FF_, NU_, LPR_, D_) \
    if (p.wfmt == F_ && a.F == FF_) return t1_launch_dn<F_, NU_, LPR_, D_>(a, grid_dn, 512, ld, s);
    // ffn 2048: 4 expert slots in flight, refilled as each is consumed (with
    // all 8 requested at once the first burst ran 1.3% slower for Q2K and 3%
    // for MXFP4 and Q4K: more requests than the memory system serves without
    // queueing them)
    T1_DN(1, 1024, 1, 16, 8) T1_DN(1, 2048, 1, 32, 4)
    T1_DN(2, 1024, 2, 16, 8) T1_DN(2, 2048, 2, 32, 4)
    T1_DN(4, 2048, 1, 32, 4)
#undef T1_DN
    return hipErrorInvalidValue;
}

}  // namespace ds4
