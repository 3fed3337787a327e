// Router top-k (one wave64 per token, shuffle argmax) and the token-to-expert
// permutation (LDS histogram, LDS prefix sum, stable scatter through per-tile
// token bitmaps).
//
// Routing stays at original precision on the pages (hysenlabs
// "DwarfStar実地分析", section "GGUFの対応範囲は意図的に狭い"); the rule
// implemented -- softmax, top-k with ties to the lower index, renormalise --
// is the library's reading of the router.
#include "common.hpp"
#include "launch.hpp"

namespace ds4 {

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, o, WAVE);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, WAVE);
        const uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w > v ? w : v;
    }
    return v;
}

// KPL logits per lane (E <= 64 * KPL).
template <int KPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;
    uint64_t keys[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + WAVE * i;
        keys[i] = e < E ? route_key(row[e], e) : 0ull;
    }
    float my_logit = 0.0f;       // lane j keeps the j-th selected logit
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) best = keys[i] > best ? keys[i] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < KPL; ++i) keys[i] = keys[i] == best ? 0ull : keys[i];
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        if (lane == 0) topk_idx[(size_t)t * k + j] = e;
        if (lane == j) my_logit = key_value(best);
    }
    const float l0 = __shfl(my_logit, 0, WAVE);
    const float ex = lane < k ? expf(my_logit - l0) : 0.0f;
    const float sum = wave_sum(ex);
    if (lane < k) topk_w[(size_t)t * k + lane] = ex / sum;
}

// One 1024-thread workgroup.  LDS: cnt[E] cursor[E] bitmap[E*W] prefix[E*W]
// (W = 32-bit words of token bitmap per expert per tile, tile = 32*W tokens).
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ topk_idx, int T, int E, int k,
                                                       int W, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_pair,
                                                       int32_t* __restrict__ pair_pos,
                                                       int32_t* __restrict__ active) {
    extern __shared__ uint32_t lds[];
    int* cnt = reinterpret_cast<int*>(lds);
    int* cursor = cnt + E;
    int* tmp = cursor + E;                       // 32 ints
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(tmp + 32);
    uint16_t* prefix = reinterpret_cast<uint16_t*>(bitmap + (size_t)E * W);
    const int tid = threadIdx.x;
    const int P = T * k;

    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = topk_idx[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);    // counts only
    }
    __syncthreads();
    // offsets = exclusive scan of counts; active = ids with a count, ascending
    {
        int total = 0, n_act = 0;
        const int c = tid < E ? cnt[tid] : 0;
        const int ex = block_exclusive_scan(c, tmp, &total);
        const int rank = block_exclusive_scan(c > 0 ? 1 : 0, tmp, &n_act);
        if (tid < E) {
            offsets[tid] = ex;
            cursor[tid] = ex;
            if (c > 0) active[1 + rank] = tid;
        }
        if (tid == 0) {
            offsets[E] = total;
            active[0] = n_act;
        }
    }
    __syncthreads();
    const int TT = 32 * W;
    for (int t0 = 0; t0 < T; t0 += TT) {
        for (int i = tid; i < E * W; i += blockDim.x) bitmap[i] = 0u;
        __syncthreads();
        const int t = t0 + tid;
        const bool mine = tid < TT && t < T;
        if (mine) {
            for (int j = 0; j < k; ++j) {
                const int e = topk_idx[(size_t)t * k + j];
                if ((unsigned)e < (unsigned)E) atomicOr(&bitmap[e * W + (tid >> 5)], 1u << (tid & 31));
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += blockDim.x) {
            int run = 0;
            for (int w = 0; w < W; ++w) {
                prefix[e * W + w] = (uint16_t)run;
                run += __popc(bitmap[e * W + w]);
            }
            cnt[e] = run;
        }
        __syncthreads();
        if (mine) {
            const uint32_t below = (1u << (tid & 31)) - 1u;
            for (int j = 0; j < k; ++j) {
                const int e = topk_idx[(size_t)t * k + j];
                if ((unsigned)e >= (unsigned)E) continue;
                const int w = tid >> 5;
                const int r = cursor[e] + prefix[e * W + w] + __popc(bitmap[e * W + w] & below);
                if ((unsigned)r < (unsigned)P) {
                    sorted_pair[r] = t * k + j;
                    pair_pos[(size_t)t * k + j] = r;
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += blockDim.x) cursor[e] += cnt[e];
        __syncthreads();
    }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
    const dim3 grid((T + 3) / 4);
    if (E <= 64) return launch_stage(STAGE_ROUTE, route_kernel<1>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
    if (E <= 128) return launch_stage(STAGE_ROUTE, route_kernel<2>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
    if (E <= 256) return launch_stage(STAGE_ROUTE, route_kernel<4>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
    if (E <= 512) return launch_stage(STAGE_ROUTE, route_kernel<8>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
    return launch_stage(STAGE_ROUTE, route_kernel<16>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
}

// Bitmap words per expert per token tile: as few as the token count needs,
// at most 32 (1024 tokens, one per thread), LDS bitmap <= 32 KiB.
int permute_words(int E, int T) {
    int W = 8192 / E;
    if (W > 32) W = 32;
    const int need = (T + 31) / 32;
    if (W > need) W = need;
    if (W < 1) W = 1;
    return W;
}

size_t permute_lds_bytes(int E, int T) {
    const int W = permute_words(E, T);
    return (size_t)(2 * E + 32) * 4 + (size_t)E * W * 4 + (size_t)E * W * 2;
}

hipError_t launch_permute(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_pos, int32_t* active, hipStream_t s) {
    const int W = permute_words(E, T);
    // one thread per token of a tile, at least one per expert
    int threads = 32 * W > E ? 32 * W : E;
    threads = ((threads + 63) / 64) * 64;
    if (threads > 1024) threads = 1024;
    return launch_stage(STAGE_PERMUTE, permute_kernel, dim3(1), dim3(threads), permute_lds_bytes(E, T), s, idx, T, E, k,
                        W, offsets, sorted_pair, pair_pos, active);
}

// ---- blocked permutation (many tokens) ---------------------------------------------
// The same stable counting sort in three launches over blocks of PB_TOKENS
// tokens: per-block expert counts; one workgroup scanning each expert's
// column of block counts (block bases) and the expert totals (offsets, the
// active list); a per-block scatter whose rank within (block, expert) is the
// popcount of the block's token bitmap of that expert below the token.
constexpr int PB_TOKENS = 128;
constexpr int PB_WORDS = PB_TOKENS / 32;

__global__ __launch_bounds__(256) void pb_count_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                       int32_t* __restrict__ counts) {
    extern __shared__ int cnt[];
    const int b = blockIdx.x, t0 = b * PB_TOKENS;
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int nt = min(PB_TOKENS, T - t0);
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const int e = idx[(size_t)t0 * k + i];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(size_t)b * E + e] = cnt[e];
}

// One workgroup of round64(max(E, 64)) <= 1024 threads: thread e walks its
// column; base[b][e] = pairs of expert e in blocks before b.
__global__ __launch_bounds__(1024) void pb_scan_kernel(const int32_t* __restrict__ counts, int B, int E,
                                                       int32_t* __restrict__ base, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ active) {
    __shared__ int tmp[32];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int b = 0; b < B; ++b) {
            const int c = counts[(size_t)b * E + e];
            base[(size_t)b * E + e] = run;
            run += c;
        }
    }
    int total = 0, n_act = 0;
    const int ex = block_exclusive_scan(run, tmp, &total);
    const int rank = block_exclusive_scan(run > 0 ? 1 : 0, tmp, &n_act);
    if (e < E) {
        offsets[e] = ex;
        if (run > 0) active[1 + rank] = e;
    }
    if (e == 0) {
        offsets[E] = total;
        active[0] = n_act;
    }
}

__global__ __launch_bounds__(256) void pb_scatter_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ base,
                                                         int32_t* __restrict__ sorted_pair,
                                                         int32_t* __restrict__ pair_pos) {
    extern __shared__ uint32_t bm[];   // [E][PB_WORDS]
    const int b = blockIdx.x, t0 = b * PB_TOKENS;
    const int P = T * k;
    for (int i = threadIdx.x; i < E * PB_WORDS; i += blockDim.x) bm[i] = 0u;
    __syncthreads();
    const int nt = min(PB_TOKENS, T - t0);
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const int e = idx[(size_t)t0 * k + i];
        const int tl = i / k;
        if ((unsigned)e < (unsigned)E) atomicOr(&bm[e * PB_WORDS + (tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const int e = idx[(size_t)t0 * k + i];
        if ((unsigned)e >= (unsigned)E) continue;
        const int tl = i / k, w = tl >> 5;
        int r = offsets[e] + base[(size_t)b * E + e];
        for (int v = 0; v < w; ++v) r += __popc(bm[e * PB_WORDS + v]);
        r += __popc(bm[e * PB_WORDS + w] & ((1u << (tl & 31)) - 1u));
        if ((unsigned)r < (unsigned)P) {
            const int p = t0 * k + i;
            sorted_pair[r] = p;
            pair_pos[p] = r;
        }
    }
}

size_t permute_scratch_bytes(int E, int T) {
    const size_t B = ((size_t)T + PB_TOKENS - 1) / PB_TOKENS;
    return 2 * B * (size_t)E * 4;
}

hipError_t launch_permute_blocked(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* sorted_pair,
                                  int32_t* pair_pos, int32_t* active, int32_t* scratch, hipStream_t s) {
    const int B = (T + PB_TOKENS - 1) / PB_TOKENS;
    int32_t* counts = scratch;
    int32_t* base = scratch + (size_t)B * E;
    hipError_t err = launch_stage(STAGE_PERMUTE, pb_count_kernel, dim3(B), dim3(256),
                                       (size_t)E * 4, s, idx, T, E, k, counts);
    if (err != hipSuccess) return err;
    const int threads = ((E > 64 ? E : 64) + 63) / 64 * 64;
    err = launch_stage(STAGE_PERMUTE, pb_scan_kernel, dim3(1), dim3(threads), 0, s, counts, B, E,
                            base, offsets, active);
    if (err != hipSuccess) return err;
    return launch_stage(STAGE_PERMUTE, pb_scatter_kernel, dim3(B), dim3(256),
                             (size_t)E * PB_WORDS * 4, s, idx, T, E, k, offsets, base, sorted_pair, pair_pos);
}

}  // namespace ds4
