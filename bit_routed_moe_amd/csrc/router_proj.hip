// Router projection: logits[t][e] = sum_h W_r[e][h] * x[t][h], fp32 logits
// from bf16 router weights [E][H].
//
// The pages keep the router (like the shared expert and the other
// projections) at original precision while only the routed experts are
// quantized (hysenlabs "DwarfStar実地分析", section
// "GGUFの対応範囲は意図的に狭い"); this library reads that as bf16 weights
// and fp32 accumulation.  bf16 x bf16 products are exact in fp32, so only
// the order of the fp32 additions differs between the two kernels.
//
//   router_gemv_kernel  (fp32 mode, or at most 16 tokens) one workgroup per
//                       (expert row, block of 16 tokens): the row is read
//                       once as 16-byte chunks, each thread keeps 16 token
//                       sums, a wave butterfly and a 4-wave LDS sum finish
//                       them.  At batch 1 this streams the E*H*2 weight bytes
//                       once (3.7 MB for 256 x 7168).
//   router_mfma_kernel  (bf16, more tokens) 64 tokens x 64 experts per
//                       workgroup on v_mfma_f32_16x16x32_bf16: wave w owns 16
//                       tokens and the four 16-expert tiles, operands loaded
//                       straight from global memory (the workgroup's four
//                       waves share the weight tile through the caches).
#include "common.hpp"
#include "launch.hpp"

namespace ds4 {

namespace {

constexpr int RG_TOK = 16;        // tokens per GEMV workgroup
constexpr int RG_CPT = 4;         // row chunks per thread and pass (rows up to 8192 in one pass)
constexpr int RG_THREADS = 256;
constexpr int RM_TILE = 64;       // tokens and experts per MFMA workgroup
constexpr int RM_KB = 4;          // k-steps (of 32) per operand block

__device__ __forceinline__ void unpack_bf16x8(const u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
    }
}

// grid (ceil(T / 16), E): x blocks of 16 tokens fastest, so the workgroups
// of one expert row run back to back and share the row in the cache.
template <bool F32X>
__global__ __launch_bounds__(RG_THREADS) void router_gemv_kernel(const uint16_t* __restrict__ w,
                                                                 const void* __restrict__ x, int T, int H, int E,
                                                                 float* __restrict__ logits) {
    const int t0 = blockIdx.x * RG_TOK;
    const int e = blockIdx.y;
    const int nt = min(RG_TOK, T - t0);
    const u32x4* wr = reinterpret_cast<const u32x4*>(w + (size_t)e * H);
    float acc[RG_TOK];
#pragma unroll
    for (int j = 0; j < RG_TOK; ++j) acc[j] = 0.0f;
    const int nch = H / 8;   // 16-byte chunks of 8 weights
    // all of a pass's row chunks are requested before the first is used (a
    // 7168-wide row is one pass), so the row costs one memory round trip
    for (int c0 = threadIdx.x; c0 < nch; c0 += RG_THREADS * RG_CPT) {
        u32x4 wv[RG_CPT];
#pragma unroll
        for (int u = 0; u < RG_CPT; ++u) {
            const int c = c0 + u * RG_THREADS;
            wv[u] = wr[c < nch ? c : c0];
        }
#pragma unroll
        for (int u = 0; u < RG_CPT; ++u) {
            const int c = c0 + u * RG_THREADS;
            if (c >= nch) break;
            float wf[8];
            unpack_bf16x8(wv[u], wf);
#pragma unroll
            for (int j = 0; j < RG_TOK; ++j) {
                if (j < nt) {
                    float xf[8];
                    if constexpr (F32X) {
                        const f32x4* xr = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) +
                                                                         (size_t)(t0 + j) * H) + 2 * c;
                        const f32x4 a = xr[0], b = xr[1];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            xf[i] = a[i];
                            xf[4 + i] = b[i];
                        }
                    } else {
                        const u32x4* xr = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) +
                                                                         (size_t)(t0 + j) * H);
                        unpack_bf16x8(xr[c], xf);
                    }
                    float s = acc[j];
#pragma unroll
                    for (int i = 0; i < 8; ++i) s = fmaf(wf[i], xf[i], s);
                    acc[j] = s;
                }
            }
        }
    }
    __shared__ float red[RG_THREADS / WAVE][RG_TOK];
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
#pragma unroll
    for (int j = 0; j < RG_TOK; ++j) {
        if (j < nt) {
            const float v = wave_sum(acc[j]);
            if (lane == 0) red[wave][j] = v;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < nt) {
        const int j = threadIdx.x;
        float s = red[0][j];
#pragma unroll
        for (int q = 1; q < RG_THREADS / WAVE; ++q) s += red[q][j];
        logits[(size_t)(t0 + j) * E + e] = s;
    }
}

// grid (ceil(T / 64), ceil(E / 64)).  Lane l of a wave supplies row l % 16 of
// each operand tile with the 8 consecutive k values from 8 * (l / 16) of the
// 32-wide step (the same lane -> k map for both operands, so the product is
// the full dot product), and receives C[4 * (l / 16) + i][l % 16] of each
// 16 x 16 tile: experts along rows, tokens along columns.  Rows past T or E
// read the last valid row and are not stored.
__global__ __launch_bounds__(RG_THREADS) void router_mfma_kernel(const uint16_t* __restrict__ w,
                                                                 const uint16_t* __restrict__ x, int T, int H, int E,
                                                                 float* __restrict__ logits) {
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int m = lane & 15, q4 = lane >> 4;
    const int t0 = blockIdx.x * RM_TILE + 16 * wv;
    const int e0 = blockIdx.y * RM_TILE;
    const uint16_t* xr = x + (size_t)min(t0 + m, T - 1) * H + 8 * q4;
    const uint16_t* wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[i] = w + (size_t)min(e0 + 16 * i + m, E - 1) * H + 8 * q4;
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // operands of RM_KB k-steps at a time, the next block requested before
    // the current one is multiplied (H % (32 * RM_KB) == 0; the last block
    // requests itself again, in bounds)
    bf16x8 xa[RM_KB], wa[RM_KB][4];
    auto load = [&](int k0, bf16x8 (&xb)[RM_KB], bf16x8 (&wb)[RM_KB][4]) {
#pragma unroll
        for (int s = 0; s < RM_KB; ++s) {
            xb[s] = *reinterpret_cast<const bf16x8*>(xr + k0 + 32 * s);
#pragma unroll
            for (int i = 0; i < 4; ++i) wb[s][i] = *reinterpret_cast<const bf16x8*>(wrow[i] + k0 + 32 * s);
        }
    };
    load(0, xa, wa);
    for (int k0 = 0; k0 < H; k0 += 32 * RM_KB) {
        bf16x8 xn[RM_KB], wn[RM_KB][4];
        load(k0 + 32 * RM_KB < H ? k0 + 32 * RM_KB : k0, xn, wn);
#pragma unroll
        for (int s = 0; s < RM_KB; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[s][i], xa[s], acc[i], 0, 0, 0);
#pragma unroll
        for (int s = 0; s < RM_KB; ++s) {
            xa[s] = xn[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) wa[s][i] = wn[s][i];
        }
    }
    const int t = t0 + m;
    if (t < T) {
        float* out = logits + (size_t)t * E;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = e0 + 16 * i + 4 * q4 + j;
                if (e < E) out[e] = acc[i][j];
            }
    }
}

}  // namespace

hipError_t launch_router_logits(const void* x, bool f32x, const uint16_t* w, int T, int H, int E, float* logits,
                                hipStream_t s) {
    if (f32x || T <= RG_TOK) {
        const dim3 grid((T + RG_TOK - 1) / RG_TOK, E);
        if (f32x)
            return launch_stage(STAGE_ROUTER_PROJ, router_gemv_kernel<true>, grid, dim3(RG_THREADS), 0, s, w, x, T,
                                H, E, logits);
        return launch_stage(STAGE_ROUTER_PROJ, router_gemv_kernel<false>, grid, dim3(RG_THREADS), 0, s, w, x, T, H,
                            E, logits);
    }
    const dim3 grid((T + RM_TILE - 1) / RM_TILE, (E + RM_TILE - 1) / RM_TILE);
    return launch_stage(STAGE_ROUTER_PROJ, router_mfma_kernel, grid, dim3(RG_THREADS), 0, s, w,
                        static_cast<const uint16_t*>(x), T, H, E, logits);
}

}  // namespace ds4
