// Native driver for libds4moe without Python, for hardware-counter runs.
//
//   ds4moe_bench <workload> [steps] [warmup] [copies]
//   ds4moe_bench copy <MiB> [reps]
//   ds4moe_bench router_decode | router_prefill [steps] [warmup] [copies]
//
// <workload>: tiny | decode | batched_decode | prefill | mxfp4_decode |
// mxfp4_prefill | mxfp4_prefill_fp8 (MXFP8 x and h on the scaled matrix
// instructions) | q4k_decode | q4k_prefill, the same shapes as the Python
// benchmark.  The layer lives on
// the device, filled by counter-hash kernels: Q2K blocks with uniform code and
// scale bytes and fp16 d / dmin in the range a N(0, 0.02) matrix quantizes to;
// MXFP4 codes uniform with E8M0 scales 2^-10 .. 2^-6; bf16 shared weights
// uniform in +-0.04; activations uniform in +-2; router logits uniform in
// +-2 (batched_decode adds a Zipf(1.1) popularity bias per expert).  Layer
// copies and 8 logit draws rotate per step.  Prints one line with the
// average ms per ds4moe_forward step (HIP events on the stream).
//
// router_decode / router_prefill time ds4moe_router_logits alone (7168
// hidden, 256 experts, 1 or 4096 tokens; bf16 router matrices uniform in
// +-0.02 rotating over 96 or 2 copies, activations uniform in +-2).
//
// `copy` runs a plain device copy of <MiB> MiB (16-byte loads and stores),
// whose memory counters (FETCH_SIZE, WRITE_SIZE) per dispatch calibrate those
// of the layer kernels against known byte counts.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ds4moe.h"

#define CHECK(x)                                                                                 \
    do {                                                                                         \
        hipError_t e_ = (x);                                                                     \
        if (e_ != hipSuccess) {                                                                  \
            fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            exit(1);                                                                             \
        }                                                                                        \
    } while (0)

#define CHECK_DS(x)                                                                           \
    do {                                                                                      \
        int s_ = (x);                                                                         \
        if (s_ != DS4MOE_OK) {                                                                \
            fprintf(stderr, "ds4moe error %d (%s) at line %d\n", s_, ds4moe_last_error(), __LINE__); \
            exit(1);                                                                          \
        }                                                                                     \
    } while (0)

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ float unit(uint64_t h) { return (float)(h >> 40) * (1.0f / 16777216.0f); }

__global__ void fill_bytes(uint8_t* p, size_t n, uint64_t seed) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = (uint8_t)mix64(seed ^ (i * 0x2545F4914F6CDD1Dull));
}
// Q2K: 84-byte blocks; scale/min nibbles and codes uniform, fp16 d and dmin
// around 1.3e-3 and 1.7e-3.
__global__ void fill_q2k(uint8_t* p, size_t nblocks, uint64_t seed) {
    for (size_t b = blockIdx.x * (size_t)blockDim.x + threadIdx.x; b < nblocks; b += (size_t)gridDim.x * blockDim.x) {
        uint8_t* blk = p + b * 84;
        for (int i = 0; i < 80; i += 8) {
            const uint64_t h = mix64(seed ^ (b * 0x9E3779B97F4A7C15ull) ^ (uint64_t)i);
            memcpy(blk + i, &h, 8);
        }
        const uint64_t h = mix64(seed ^ ~b);
        const _Float16 d = (_Float16)(1.0e-3f + 0.6e-3f * unit(h));
        const _Float16 dm = (_Float16)(1.3e-3f + 0.8e-3f * unit(mix64(h)));
        memcpy(blk + 80, &d, 2);
        memcpy(blk + 82, &dm, 2);
    }
}
// Q4K parameter records (20 bytes per 256 weights): scale/min nibbles
// uniform, fp16 d and dmin around 0.5e-3 and 1.8e-3.
__global__ void fill_q4k_params(uint8_t* p, size_t nrec, uint64_t seed) {
    for (size_t b = blockIdx.x * (size_t)blockDim.x + threadIdx.x; b < nrec; b += (size_t)gridDim.x * blockDim.x) {
        uint8_t* rec = p + b * 20;
        for (int i = 0; i < 16; i += 8) {
            const uint64_t h = mix64(seed ^ (b * 0x9E3779B97F4A7C15ull) ^ (uint64_t)i);
            memcpy(rec + i, &h, 8);
        }
        const uint64_t h = mix64(seed ^ ~b);
        const _Float16 d = (_Float16)(0.4e-3f + 0.2e-3f * unit(h));
        const _Float16 dm = (_Float16)(1.3e-3f + 0.8e-3f * unit(mix64(h)));
        memcpy(rec + 16, &d, 2);
        memcpy(rec + 18, &dm, 2);
    }
}
__global__ void fill_e8m0(uint8_t* p, size_t n, uint64_t seed) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = (uint8_t)(117 + mix64(seed ^ i) % 5);
}
__global__ void fill_bf16(uint16_t* p, size_t n, uint64_t seed, float scale) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const float v = (2.0f * unit(mix64(seed ^ i)) - 1.0f) * scale;
        const __bf16 b = (__bf16)v;
        p[i] = __builtin_bit_cast(uint16_t, b);
    }
}
__global__ void fill_logits(float* p, int T, int E, uint64_t seed, float zipf) {
    const size_t n = (size_t)T * E;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const int e = (int)(i % E);
        const float bias = zipf > 0.0f ? -zipf * logf((float)(e + 1)) : 0.0f;
        p[i] = (2.0f * unit(mix64(seed ^ i)) - 1.0f) * 2.0f + bias;
    }
}
__global__ void copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

struct Shape {
    const char* name;
    int H, F, E, k, Fs, wfmt, T;
    float zipf;
    int mma;
};
static const Shape SHAPES[] = {
    {"tiny", 256, 128, 8, 2, 0, DS4MOE_WFMT_Q2K, 16, 0.0f, DS4MOE_DT_BF16},
    {"decode", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_Q2K, 1, 0.0f, DS4MOE_DT_BF16},
    {"batched_decode", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_Q2K, 32, 1.1f, DS4MOE_DT_BF16},
    {"prefill", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_Q2K, 4096, 0.0f, DS4MOE_DT_BF16},
    {"mxfp4_decode", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_MXFP4, 1, 0.0f, DS4MOE_DT_BF16},
    {"mxfp4_prefill", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_MXFP4, 4096, 0.0f, DS4MOE_DT_BF16},
    {"mxfp4_prefill_fp8", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_MXFP4, 4096, 0.0f, DS4MOE_DT_FP8_E4M3},
    {"q4k_decode", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_Q4K, 1, 0.0f, DS4MOE_DT_BF16},
    {"q4k_prefill", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_Q4K, 4096, 0.0f, DS4MOE_DT_BF16},
    {"verify6", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_Q2K, 6, 0.0f, DS4MOE_DT_BF16},
    {"sessions16", 7168, 2048, 256, 8, 2048, DS4MOE_WFMT_Q2K, 16, 1.1f, DS4MOE_DT_BF16},
};

static void* dalloc(size_t bytes) {
    void* p = nullptr;
    CHECK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}
static const int FILL_GRID = 4096, FILL_BLOCK = 256;

// Read-only stream: each thread reads its 16-byte pieces of a region, U in
// flight per iteration, and folds them into one word that it writes once, so
// the reads are live: the plain HBM read rate that the weight streams are
// measured against (run_stream reports six grid and depth settings).  Dispatch r reads region r % regions, so that with a
// region per dispatch no smaller than the launch it stands for and regions
// whose sum exceeds the 256 MB cache, every dispatch reads from HBM.
template <int U>
__global__ void read16(const uint4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[blockIdx.x * (size_t)blockDim.x + threadIdx.x] = acc;
}

static int run_stream(int mib, int reps, int regions) {
    const size_t bytes = (size_t)mib << 20;
    uint8_t* a = (uint8_t*)dalloc(bytes * regions);
    hipLaunchKernelGGL(fill_bytes, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, a, bytes * regions, 9ull);
    CHECK(hipDeviceSynchronize());
    for (int cfg = 0; cfg < 6; ++cfg) {
        const int grid = cfg % 3 == 0 ? 1024 : (cfg % 3 == 1 ? 512 : 2048), U = cfg < 3 ? 4 : 8, BL = 512;
        void (*kern)(const uint4*, size_t, uint32_t*) = U == 4 ? read16<4> : read16<8>;
        uint32_t* sink = (uint32_t*)dalloc((size_t)grid * BL * 4);
        for (int r = 0; r < regions; ++r)   // warm-up pass over every region
            hipLaunchKernelGGL(kern, dim3(grid), dim3(BL), 0, 0, (const uint4*)(a + r * bytes), bytes / 16, sink);
        hipEvent_t e0, e1;
        CHECK(hipEventCreate(&e0));
        CHECK(hipEventCreate(&e1));
        CHECK(hipEventRecord(e0, 0));
        for (int r = 0; r < reps; ++r)
            hipLaunchKernelGGL(kern, dim3(grid), dim3(BL), 0, 0, (const uint4*)(a + (r % regions) * bytes),
                               bytes / 16, sink);
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        printf("read16<%d>: %zu bytes read per dispatch from %d regions, grid %d x %d, %d dispatches, "
               "%.3f us each (%.1f GB/s)\n",
               U, bytes, regions, grid, BL, reps, ms * 1e3 / reps, (double)bytes * reps / (ms * 1e-3) / 1e9);
        CHECK(hipEventDestroy(e0));
        CHECK(hipEventDestroy(e1));
    }
    return 0;
}

static int run_copy(int mib, int reps) {
    const size_t bytes = (size_t)mib << 20;
    uint4 *a = (uint4*)dalloc(bytes), *b = (uint4*)dalloc(bytes);
    hipLaunchKernelGGL(fill_bytes, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, (uint8_t*)a, bytes, 7ull);
    CHECK(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0, 0));
    for (int r = 0; r < reps; ++r)
        hipLaunchKernelGGL(copy16, dim3(2048), dim3(256), 0, 0, a, b, bytes / 16);
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("copy16: %zu bytes read + %zu bytes written per dispatch, %d dispatches, %.3f us each (%.1f GB/s)\n",
           bytes, bytes, reps, ms * 1e3 / reps, 2.0 * bytes * reps / (ms * 1e-3) / 1e9);
    return 0;
}

static int run_router(bool decode, int steps, int warmup, int copies) {
    const int H = 7168, E = 256, T = decode ? 1 : 4096;
    if (copies < 1) copies = decode ? 96 : 2;
    if (steps < 1 || warmup < 0) return 2;
    ds4moe_config cfg = {H, 2048, E, 8, 2048, DS4MOE_WFMT_Q2K, DS4MOE_DT_BF16, DS4MOE_DT_BF16, DS4MOE_ALGO_AUTO};
    std::vector<uint16_t*> wr(copies);
    for (int c = 0; c < copies; ++c) {
        wr[c] = (uint16_t*)dalloc((size_t)E * H * 2);
        hipLaunchKernelGGL(fill_bf16, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, wr[c], (size_t)E * H, 9000ull + c, 0.02f);
    }
    uint16_t* x = (uint16_t*)dalloc((size_t)T * H * 2);
    hipLaunchKernelGGL(fill_bf16, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, x, (size_t)T * H, 43ull, 2.0f);
    float* logits = (float*)dalloc((size_t)T * E * 4);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    hipStream_t s;
    CHECK(hipStreamCreate(&s));
    for (int i = 0; i < warmup; ++i) CHECK_DS(ds4moe_router_logits(&cfg, T, x, wr[i % copies], logits, s));
    CHECK(hipStreamSynchronize(s));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0, s));
    for (int i = 0; i < steps; ++i)
        CHECK_DS(ds4moe_router_logits(&cfg, T, x, wr[(warmup + i) % copies], logits, s));
    CHECK(hipEventRecord(e1, s));
    CHECK(hipEventSynchronize(e1));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("router_%s: T=%d H=%d E=%d, %d steps x %d router copies: %.4f ms/step, %.1f tokens/s\n",
           decode ? "decode" : "prefill", T, H, E, steps, copies, ms / steps, T / (ms / steps * 1e-3));
    return 0;
}

int main(int argc, char** argv) {
    if (argc < 2) {
        fprintf(stderr,
                "usage: %s <workload> [steps] [warmup] [copies] [tokens] [auto|gemv|grouped] | copy <MiB> [reps]"
                " | stream <MiB per dispatch> [reps] [regions]\n",
                argv[0]);
        return 2;
    }
    const std::string wl = argv[1];
    if (wl == "copy") return run_copy(argc > 2 ? atoi(argv[2]) : 1024, argc > 3 ? atoi(argv[3]) : 5);
    if (wl == "stream")
        return run_stream(argc > 2 ? atoi(argv[2]) : 1024, argc > 3 ? atoi(argv[3]) : 20,
                          argc > 4 ? atoi(argv[4]) : 4);
    if (wl == "router_decode" || wl == "router_prefill")
        return run_router(wl == "router_decode", argc > 2 ? atoi(argv[2]) : 20, argc > 3 ? atoi(argv[3]) : 3,
                          argc > 4 ? atoi(argv[4]) : 0);
    const Shape* sh = nullptr;
    for (const Shape& s : SHAPES)
        if (wl == s.name) sh = &s;
    if (!sh) {
        fprintf(stderr, "unknown workload %s\n", wl.c_str());
        return 2;
    }
    const int steps = argc > 2 ? atoi(argv[2]) : 20;
    const int warmup = argc > 3 ? atoi(argv[3]) : 3;
    const int copies = argc > 4 ? atoi(argv[4]) : (sh->T <= 64 ? 8 : 2);
    if (steps < 1 || warmup < 0 || copies < 1) return 2;

    // optional overrides: token count, expert-FFN algorithm
    const int T = argc > 5 && atoi(argv[5]) > 0 ? atoi(argv[5]) : sh->T;
    int algo = DS4MOE_ALGO_AUTO;
    if (argc > 6) {
        const std::string al = argv[6];
        if (al == "gemv") algo = DS4MOE_ALGO_GEMV;
        else if (al == "grouped") algo = DS4MOE_ALGO_GROUPED;
        else if (al != "auto") return 2;
    }
    ds4moe_config cfg = {sh->H, sh->F, sh->E, sh->k, sh->Fs, sh->wfmt, DS4MOE_DT_BF16, sh->mma, algo};
    const size_t HF = (size_t)sh->H * sh->F;
    const bool q2k = sh->wfmt == DS4MOE_WFMT_Q2K, q4k = sh->wfmt == DS4MOE_WFMT_Q4K;
    const size_t mat_bytes = q2k ? HF / 256 * 84 : HF / 2;
    const size_t sc_bytes = q2k ? 0 : (q4k ? HF / 256 * 20 : HF / 32);
    std::vector<ds4moe_weights> ws(copies);
    for (int c = 0; c < copies; ++c) {
        const void* mats[3];
        const void* scs[3] = {nullptr, nullptr, nullptr};
        for (int m = 0; m < 3; ++m) {
            uint8_t* d = (uint8_t*)dalloc(mat_bytes * sh->E);
            const uint64_t seed = 1000ull * c + m;
            if (q2k)
                hipLaunchKernelGGL(fill_q2k, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, d, mat_bytes * sh->E / 84, seed);
            else
                hipLaunchKernelGGL(fill_bytes, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, d, mat_bytes * sh->E, seed);
            mats[m] = d;
            if (!q2k) {
                uint8_t* s = (uint8_t*)dalloc(sc_bytes * sh->E);
                if (q4k)
                    hipLaunchKernelGGL(fill_q4k_params, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, s,
                                       sc_bytes * sh->E / 20, seed + 7);
                else
                    hipLaunchKernelGGL(fill_e8m0, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, s, sc_bytes * sh->E, seed + 7);
                scs[m] = s;
            }
        }
        const void* shm[3] = {nullptr, nullptr, nullptr};
        if (sh->Fs > 0)
            for (int m = 0; m < 3; ++m) {
                uint16_t* d = (uint16_t*)dalloc((size_t)sh->H * sh->Fs * 2);
                hipLaunchKernelGGL(fill_bf16, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, d, (size_t)sh->H * sh->Fs,
                                   5000ull * c + m, 0.04f);
                shm[m] = d;
            }
        ws[c] = ds4moe_weights{mats[0], mats[1], mats[2], scs[0], scs[1], scs[2], shm[0], shm[1], shm[2]};
    }
    CHECK(hipGetLastError());
    uint16_t* x = (uint16_t*)dalloc((size_t)T * sh->H * 2);
    hipLaunchKernelGGL(fill_bf16, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, x, (size_t)T * sh->H, 42ull, 2.0f);
    const int NL = 8;
    std::vector<float*> logits(NL);
    for (int i = 0; i < NL; ++i) {
        logits[i] = (float*)dalloc((size_t)T * sh->E * 4);
        hipLaunchKernelGGL(fill_logits, dim3(FILL_GRID), dim3(FILL_BLOCK), 0, 0, logits[i], T, sh->E, 77ull + i,
                           sh->zipf);
    }
    uint16_t* y = (uint16_t*)dalloc((size_t)T * sh->H * 2);
    const size_t wsb = ds4moe_workspace_bytes(&cfg, T);
    if (wsb == 0) {
        fprintf(stderr, "invalid config\n");
        return 1;
    }
    void* wsp = dalloc(wsb);
    CHECK(hipDeviceSynchronize());

    hipStream_t s;
    CHECK(hipStreamCreate(&s));
    for (int i = 0; i < warmup; ++i)
        CHECK_DS(ds4moe_forward(&cfg, &ws[i % copies], T, x, logits[i % NL], y, wsp, wsb, s));
    CHECK(hipStreamSynchronize(s));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0, s));
    for (int i = 0; i < steps; ++i)
        CHECK_DS(ds4moe_forward(&cfg, &ws[(warmup + i) % copies], T, x, logits[(warmup + i) % NL], y, wsp, wsb, s));
    CHECK(hipEventRecord(e1, s));
    CHECK(hipEventSynchronize(e1));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("%s: T=%d H=%d F=%d E=%d k=%d Fs=%d %s, %d steps x %d layer copies: %.4f ms/step, %.1f tokens/s\n",
           sh->name, T, sh->H, sh->F, sh->E, sh->k, sh->Fs, q2k ? "q2k" : (q4k ? "q4k" : "mxfp4"), steps, copies,
           ms / steps,
           T / (ms / steps * 1e-3));
    return 0;
}
