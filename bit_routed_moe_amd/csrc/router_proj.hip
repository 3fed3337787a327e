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
//                       workgroup on v_mfma_f32_16x16x32_bf16, both operand
//                       tiles brought into a 4-deep LDS ring 128 k-columns
//                       at a time by direct-to-LDS loads and read there by
//                       the four waves (32 x 32 each).
#include "common.hpp"
#include "launch.hpp"

namespace ds4 {

namespace {

constexpr int RG_TOK = 16;        // tokens per GEMV workgroup
constexpr int RG_CPT = 4;         // row chunks per thread and pass (rows up to 8192 in one pass)
constexpr int RG_THREADS = 256;
constexpr int RM_TILE = 64;       // experts per MFMA workgroup
constexpr int RM_TT = 64;         // tokens per MFMA workgroup
constexpr int RM_WT = RM_TT / 32;  // 16-token tiles per wave
constexpr int RM_KS = 128;        // k-columns per LDS stage (H % 128 == 0)

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

// 64 lanes x 16 bytes from global memory straight into LDS at lds_dst + 16 *
// lane (no registers on the way).  Issued as inline asm so that the
// compiler's wait-count pass leaves the LDS reads alone; the stage loop waits
// for the DMAs explicitly.
__device__ __forceinline__ void rm_dma16(const void* g, uint32_t lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are outstanding
// (loads and DMAs complete in issue order).
template <int N>
__device__ __forceinline__ void rm_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// grid (ceil(T / 64), ceil(E / 64)).  Each stage is 128 k-columns of the
// workgroup's 64 expert rows and 64 token rows (32 KiB), brought into a ring
// of RM_NS stage buffers by global_load_lds_dwordx4, RM_NS - 1 stages ahead
// (96 KiB in flight per CU, no registers held for it).  In a buffer, row r
// holds its 16 chunks of 16 bytes with chunk c in slot c ^ (r & 15): the
// fragment reads of 16 rows at one chunk then cover all 64 banks.  Each wave
// issues 8 DMAs per stage (4 of expert rows, 4 of token rows; DMA i covers
// rows 4i .. 4i+3), every stage the same, past the last stage the last stage
// again into a buffer no longer read, so the waits are compile-time counts.
// One barrier per stage: after it, stage st has landed for every wave and
// every wave is done with stage st - 1, whose buffer the next request fills.
// 64 x 64 tiles keep the operand bytes read through the caches near their
// minimum for a grid that covers the chip: the router matrix is read once
// per token tile and x once per expert tile.  Wave w computes experts
// 32 * (w & 1) .. +31 x tokens 32 * (w >> 1) .. +31 as 2 x 2 tiles of
// 16 x 16.  Lane l supplies row l % 16 of each operand tile with the 8
// consecutive k values from 8 * (l / 16) of the 32-wide step (the same
// lane -> k map for both operands, so the product is the full dot product),
// and receives C[4 * (l / 16) + i][l % 16] of each 16 x 16 tile: experts
// along rows, tokens along columns.  Rows past T or E read the last valid
// row and are not stored.
constexpr int RM_NS = 4;                          // stage buffers
constexpr int RM_ROWB = RM_KS * 2;                // bytes per staged row
constexpr int RM_OPB = RM_TILE * RM_ROWB;         // one operand's stage: 16 KiB
constexpr int RM_STB = 2 * RM_OPB;                // one stage buffer: 32 KiB
constexpr int RM_DMA_W = RM_TILE / 4 / 4;         // expert-row DMAs per wave and stage
static_assert(RM_TILE == RM_TT && RM_TILE % 16 == 0 && RM_DMA_W == 4, "4 rows per DMA, 4 waves");
__global__ __launch_bounds__(RG_THREADS) void router_mfma_kernel(const uint16_t* __restrict__ w,
                                                                 const uint16_t* __restrict__ x, int T, int H, int E,
                                                                 float* __restrict__ logits) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[RM_NS * RM_STB];
    const uint32_t lds32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int ws = __builtin_amdgcn_readfirstlane(wv);
    const int m = lane & 15, q4 = lane >> 4;
    const int t0 = blockIdx.x * RM_TT, e0 = blockIdx.y * RM_TILE;
    // DMA i of this wave (i < 4: expert rows, else token rows) covers operand
    // rows r = 4 * (4 * ws + i % 4) + lane / 16; the lane fetches chunk
    // (lane % 16) ^ (r & 15) of its row into slot lane % 16
    const uint16_t* src[2 * RM_DMA_W];
#pragma unroll
    for (int i = 0; i < 2 * RM_DMA_W; ++i) {
        const int r = 4 * (4 * ws + i % RM_DMA_W) + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        src[i] = i < RM_DMA_W ? w + (size_t)min(e0 + r, E - 1) * H + 8 * c
                              : x + (size_t)min(t0 + r, T - 1) * H + 8 * c;
    }
    const int nst = H / RM_KS;
    auto issue = [&](int st) {
        const int sc = min(st, nst - 1);
        const uint32_t buf = lds32 + (uint32_t)(st % RM_NS) * RM_STB;
#pragma unroll
        for (int i = 0; i < 2 * RM_DMA_W; ++i)
            rm_dma16(src[i] + sc * RM_KS,
                     buf + (i < RM_DMA_W ? 0u : (uint32_t)RM_OPB) + (uint32_t)(4 * ws + i % RM_DMA_W) * 1024u);
    };
    const int ea = 32 * (wv & 1), ta = 16 * RM_WT * (wv >> 1);
    f32x4 acc[2][RM_WT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < RM_WT; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < RM_NS - 1; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
        rm_wait_vm<(RM_NS - 2) * 2 * RM_DMA_W>();   // this wave's DMAs of stage st are in
        __syncthreads();
        issue(st + RM_NS - 1);                      // into the buffer of stage st - 1
        const uint8_t* lw = lds + (st % RM_NS) * RM_STB;
        const uint8_t* lx = lw + RM_OPB;
#pragma unroll
        for (int ks = 0; ks < RM_KS / 32; ++ks) {
            const int slot = ((4 * ks + q4) ^ m) << 4;   // rows 16 i + m: (row & 15) == m
            bf16x8 bt[RM_WT];
#pragma unroll
            for (int j = 0; j < RM_WT; ++j)
                bt[j] = *reinterpret_cast<const bf16x8*>(lx + (ta + 16 * j + m) * RM_ROWB + slot);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(lw + (ea + 16 * i + m) * RM_ROWB + slot);
#pragma unroll
                for (int j = 0; j < RM_WT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bt[j], acc[i][j], 0, 0, 0);
            }
        }
    }
    rm_wait_vm<0>();   // no DMA may still target LDS when the workgroup ends
#pragma unroll
    for (int j = 0; j < RM_WT; ++j) {
        const int t = t0 + ta + 16 * j + m;
        if (t >= T) continue;
        float* out = logits + (size_t)t * E;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = e0 + ea + 16 * i + 4 * q4 + r;
                if (e < E) out[e] = acc[i][j][r];
            }
    }
}

}  // namespace

hipError_t launch_router_logits(const void* x, bool f32x, const uint16_t* w, int T, int H, int E, float* logits,
                                hipStream_t s) {
    // whole 16-byte row chunks; the matrix-core kernel's stage loop also
    // takes an even number of 128-column stages
    if (T < 1 || E < 1 || H < 256 || H % 256 != 0) return hipErrorInvalidValue;
    if (f32x || T <= RG_TOK) {
        const dim3 grid((T + RG_TOK - 1) / RG_TOK, E);
        if (f32x)
            return launch_stage(STAGE_ROUTER_PROJ, router_gemv_kernel<true>, grid, dim3(RG_THREADS), 0, s, w, x, T,
                                H, E, logits);
        return launch_stage(STAGE_ROUTER_PROJ, router_gemv_kernel<false>, grid, dim3(RG_THREADS), 0, s, w, x, T, H,
                            E, logits);
    }
    const dim3 grid((T + RM_TT - 1) / RM_TT, (E + RM_TILE - 1) / RM_TILE);
    return launch_stage(STAGE_ROUTER_PROJ, router_mfma_kernel, grid, dim3(RG_THREADS), 0, s, w,
                        static_cast<const uint16_t*>(x), T, H, E, logits);
}

}  // namespace ds4
