// fp32 mode expert FFN, the dequantize test export, and the weighted combine.
//
// fp32 mode decodes every weight to its exact fp32 value (formats.hpp) and
// runs fp32 FMA against fp32 activations.  It is the reference-precision mode
// of the library: one workgroup per (expert, 16-row tile), the expert's tokens
// staged into LDS a few at a time.  Performance is not its purpose.
#include "formats.hpp"
#include "launch.hpp"

namespace ds4 {

constexpr int F32_TC = 8;       // max tokens per LDS chunk
constexpr int F32_ROWS = 16;    // output rows per workgroup tile (4 per wave)

struct F32Geom {
    int K, rows, tiles;         // routed matrices
    int Ks, rows_s, tiles_s;    // shared expert (tiles_s = 0: none)
    int tc;                     // tokens per LDS chunk
};

template <bool UP>
__global__ __launch_bounds__(256) void ffn_f32_kernel(FfnArgs a, F32Geom g) {
    extern __shared__ float xs[];   // [tc][K]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n_active = active_count(a.active, a.E, a.T * a.k);
    const int routed_items = n_active * g.tiles;
    const int total = routed_items + g.tiles_s;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const bool routed = item < routed_items;
        int rt, row0 = 0, ntok, K, rows, fmt;
        const uint8_t *m0, *m1 = nullptr, *s0 = nullptr, *s1 = nullptr;
        if (routed) {
            const int e = a.active[1 + item / g.tiles];
            rt = item % g.tiles;
            if (!expert_rows(a.offsets, e, a.E, a.T * a.k, row0, ntok)) continue;
            K = g.K;
            rows = g.rows;
            fmt = a.wfmt;
            const size_t ds = expert_data_stride(a.wfmt, rows, K);
            const size_t ss = expert_scale_stride(a.wfmt, rows, K);
            if (UP) {
                m0 = a.gate + e * ds;
                m1 = a.up + e * ds;
                if (fmt == WFMT_MX || fmt == WFMT_Q4K) { s0 = a.gate_s + e * ss; s1 = a.up_s + e * ss; }
            } else {
                m0 = a.down + e * ds;
                if (fmt == WFMT_MX || fmt == WFMT_Q4K) s0 = a.down_s + e * ss;
            }
        } else {
            rt = item - routed_items;
            ntok = a.T;
            K = g.Ks;
            rows = g.rows_s;
            fmt = 3;
            m0 = reinterpret_cast<const uint8_t*>(UP ? a.sh_gate : a.sh_down);
            m1 = reinterpret_cast<const uint8_t*>(a.sh_up);
        }
        const int KG = K / 16;
        for (int c0 = 0; c0 < ntok; c0 += g.tc) {
            const int nt = min(g.tc, ntok - c0);
            __syncthreads();
            for (int i = threadIdx.x; i < nt * K; i += blockDim.x) {
                const int ti = i / K, col = i % K;
                const float* src;
                if (UP) {
                    const int tok = routed ? a.sorted_pair[row0 + c0 + ti] / a.k : c0 + ti;
                    src = reinterpret_cast<const float*>(a.x) + (size_t)tok * a.H;
                } else {
                    src = routed ? reinterpret_cast<const float*>(a.h) + (size_t)(row0 + c0 + ti) * a.F
                                 : reinterpret_cast<const float*>(a.sh_h) + (size_t)(c0 + ti) * a.Fs;
                }
                xs[i] = src[col];
            }
            __syncthreads();
            for (int rr = 0; rr < F32_ROWS / 4; ++rr) {
                const int r = rt * F32_ROWS + wave * (F32_ROWS / 4) + rr;
                if (r >= rows) break;                         // uniform per wave
                float acc0[F32_TC], acc1[F32_TC];
#pragma unroll
                for (int ti = 0; ti < F32_TC; ++ti) { acc0[ti] = 0.0f; acc1[ti] = 0.0f; }
                for (int gl = lane; gl < KG; gl += WAVE) {
                    float w0[16], w1[16];
                    decode_group_f32(fmt, m0, s0, (int64_t)r * KG + gl, w0);
                    if (UP) decode_group_f32(fmt, m1, s1, (int64_t)r * KG + gl, w1);
#pragma unroll
                    for (int ti = 0; ti < F32_TC; ++ti) {
                        if (ti < nt) {
                            const float* xr = xs + ti * K + gl * 16;
#pragma unroll
                            for (int c = 0; c < 16; ++c) {
                                acc0[ti] = fmaf(w0[c], xr[c], acc0[ti]);
                                if (UP) acc1[ti] = fmaf(w1[c], xr[c], acc1[ti]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int ti = 0; ti < F32_TC; ++ti) {
                    if (ti < nt) {
                        const float v0 = wave_sum(acc0[ti]);
                        if (UP) {
                            const float v1 = wave_sum(acc1[ti]);
                            if (lane == 0) {
                                const float hv = v0 / (1.0f + expf(-v0)) * v1;
                                if (routed)
                                    reinterpret_cast<float*>(a.h)[(size_t)(row0 + c0 + ti) * a.F + r] = hv;
                                else
                                    reinterpret_cast<float*>(a.sh_h)[(size_t)(c0 + ti) * a.Fs + r] = hv;
                            }
                        } else if (lane == 0) {
                            if (routed)
                                reinterpret_cast<float*>(a.expert_out)[(size_t)(row0 + c0 + ti) * a.H + r] = v0;
                            else
                                reinterpret_cast<float*>(a.shared_out)[(size_t)(c0 + ti) * a.H + r] = v0;
                        }
                    }
                }
            }
        }
    }
}

hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s) {
    const bool has_shared = a.shared_out != nullptr && a.Fs > 0;
    const int P = a.T * a.k;
    const int max_active = a.E < P ? a.E : P;
    // up: gate/up [F][H] (+ shared [Fs][H])
    {
        F32Geom g;
        g.K = a.H; g.rows = a.F; g.tiles = a.F / F32_ROWS;
        g.Ks = a.H; g.rows_s = a.Fs; g.tiles_s = has_shared ? a.Fs / F32_ROWS : 0;
        g.tc = 16384 / a.H;
        g.tc = g.tc < 1 ? 1 : (g.tc > F32_TC ? F32_TC : g.tc);
        const int items = max_active * g.tiles + g.tiles_s;
        const int grid = items < 4096 ? items : 4096;
        hipError_t err = launch_stage(STAGE_FFN_UP, ffn_f32_kernel<true>, dim3(grid), dim3(256),
                                      (size_t)g.tc * a.H * 4, s, a, g);
        if (err != hipSuccess) return err;
    }
    // down: [H][F] (+ shared [H][Fs])
    {
        F32Geom g;
        g.K = a.F; g.rows = a.H; g.tiles = a.H / F32_ROWS;
        g.Ks = a.Fs; g.rows_s = a.H; g.tiles_s = has_shared ? a.H / F32_ROWS : 0;
        const int kmax = a.F > a.Fs ? a.F : a.Fs;
        g.tc = 16384 / kmax;
        g.tc = g.tc < 1 ? 1 : (g.tc > F32_TC ? F32_TC : g.tc);
        const int items = max_active * g.tiles + g.tiles_s;
        const int grid = items < 4096 ? items : 4096;
        return launch_stage(STAGE_FFN_DOWN, ffn_f32_kernel<false>, dim3(grid), dim3(256), (size_t)g.tc * kmax * 4,
                            s, a, g);
    }
}

// ------------------------------------------------------------- dequantize ---
__global__ __launch_bounds__(256) void dequant_kernel(int wfmt, const uint8_t* __restrict__ data,
                                                      const uint8_t* __restrict__ scales, int64_t ngroups,
                                                      float* __restrict__ f32, uint16_t* __restrict__ bf16) {
    const int64_t G = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (G >= ngroups) return;
    float w[16];
    decode_group_f32(wfmt, data, scales, G, w);
    if (f32) {
#pragma unroll
        for (int c = 0; c < 16; ++c) f32[G * 16 + c] = w[c];
    }
    if (bf16) {
#pragma unroll
        for (int c = 0; c < 16; ++c) bf16[G * 16 + c] = (uint16_t)f32_to_bf16(w[c]);
    }
}

hipError_t launch_dequantize(int wfmt, const uint8_t* data, const uint8_t* scales, int64_t n, float* f32,
                             uint16_t* bf16, hipStream_t s) {
    const int64_t groups = n / 16;
    if (groups == 0) return hipSuccess;
    const int64_t blocks = (groups + 255) / 256;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, wfmt, data, scales, groups, f32,
                       bf16);
    return hipGetLastError();
}

// ---------------------------------------------------------------- combine ---
// y[t] = shared[t] + sum_j w[t][j] * expert_out[pair_pos[t*k+j]], fp32 sums in
// slot order; one thread per (token, 8 consecutive columns).  KT: the top-k
// when it is a compile-time constant (bf16): all k slot indices, then all k
// rows, are requested before the first sum, instead of one dependent pair of
// loads per slot (an invalid slot reads row 0 and is not summed).
template <bool BF16, int KT>
__global__ __launch_bounds__(256) void combine_kernel(int T, int H, int k, const void* __restrict__ eo,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ w, const void* __restrict__ so,
                                                      void* __restrict__ y) {
    const int chunks = H / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * chunks) return;
    const int t = (int)(i / chunks);
    const int c = (int)(i % chunks) * 8;
    const int P = T * k;
    float acc[8];
    if (BF16) {
        if (so) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(so) + (size_t)t * H + c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = bf16_to_f32(v[q] & 0xFFFFu);
                acc[2 * q + 1] = bf16_to_f32(v[q] >> 16);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        }
        if constexpr (KT > 0) {
            int r[KT];
            float wj[KT];
            u32x4 v[KT];
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                r[j] = pair_pos[(size_t)t * KT + j];
                wj[j] = w[(size_t)t * KT + j];
            }
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                const int rr = (unsigned)r[j] < (unsigned)P ? r[j] : 0;
                v[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(eo) + (size_t)rr * H + c);
            }
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                if ((unsigned)r[j] >= (unsigned)P) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = fmaf(wj[j], bf16_to_f32(v[j][q] & 0xFFFFu), acc[2 * q]);
                    acc[2 * q + 1] = fmaf(wj[j], bf16_to_f32(v[j][q] >> 16), acc[2 * q + 1]);
                }
            }
        } else {
            for (int j = 0; j < k; ++j) {
                const int r = pair_pos[(size_t)t * k + j];
                if ((unsigned)r >= (unsigned)P) continue;
                const float wj = w[(size_t)t * k + j];
                const u32x4 v =
                    *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(eo) + (size_t)r * H + c);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = fmaf(wj, bf16_to_f32(v[q] & 0xFFFFu), acc[2 * q]);
                    acc[2 * q + 1] = fmaf(wj, bf16_to_f32(v[q] >> 16), acc[2 * q + 1]);
                }
            }
        }
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + (size_t)t * H + c) = out;
    } else {
        const float* sp = so ? reinterpret_cast<const float*>(so) + (size_t)t * H + c : nullptr;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = sp ? sp[q] : 0.0f;
        for (int j = 0; j < k; ++j) {
            const int r = pair_pos[(size_t)t * k + j];
            if ((unsigned)r >= (unsigned)P) continue;
            const float wj = w[(size_t)t * k + j];
            const float* ep = reinterpret_cast<const float*>(eo) + (size_t)r * H + c;
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj, ep[q], acc[q]);
        }
        float* yp = reinterpret_cast<float*>(y) + (size_t)t * H + c;
#pragma unroll
        for (int q = 0; q < 8; ++q) yp[q] = acc[q];
    }
}

hipError_t launch_combine(int act_bf16, int T, int H, int k, const void* expert_out, const int32_t* pair_pos,
                          const float* topk_w, const void* shared_out, void* y, hipStream_t s) {
    const int64_t n = (int64_t)T * (H / 8);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (act_bf16 && k == 8)
        return launch_stage(STAGE_COMBINE, combine_kernel<true, 8>, dim3(blocks), dim3(256), 0, s, T, H, k,
                            expert_out, pair_pos, topk_w, shared_out, y);
    if (act_bf16)
        return launch_stage(STAGE_COMBINE, combine_kernel<true, 0>, dim3(blocks), dim3(256), 0, s, T, H, k,
                            expert_out, pair_pos, topk_w, shared_out, y);
    return launch_stage(STAGE_COMBINE, combine_kernel<false, 0>, dim3(blocks), dim3(256), 0, s, T, H, k, expert_out,
                        pair_pos, topk_w, shared_out, y);
}

}  // namespace ds4
