// Internal launcher declarations shared by the kernel translation units and
// the C-ABI host code.  Launchers enqueue on the given stream and return the
// HIP launch status; arguments are validated by the caller (api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace ds4 {

enum Stage { STAGE_ROUTE = 0, STAGE_PERMUTE = 1, STAGE_FFN_UP = 2, STAGE_FFN_DOWN = 3, STAGE_COMBINE = 4,
             STAGE_ROUTER_PROJ = 5, N_STAGES = 6 };

// Events to record around the launches of a stage on this thread (null: none).
// Within one API call the start event is taken by the stage's first launch
// and the stop event by every launch, so the interval spans all of them.
struct StageEvents {
    hipEvent_t start, stop;
};
StageEvents stage_events(int stage);
void stage_call_begin();

// Launch `kernel` for `stage`, recording the stage's events when set.
template <typename... KArgs, typename... Args>
inline hipError_t launch_stage(int stage, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                               hipStream_t s, Args... args) {
    const StageEvents ev = stage_events(stage);
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    return hipGetLastError();
}

// Everything one expert-FFN launch needs.  Routed matrices: gate/up [E][F][H],
// down [E][H][F]; per-expert byte strides follow from wfmt.  Token rows of
// expert e are sorted rows offsets[e] .. offsets[e+1]-1, token = sorted_pair/k.
struct FfnArgs {
    int H, F, Fs, E, k, T;
    int wfmt;                                   // 1 Q2K, 2 MXFP4, 4 Q4K
    const uint8_t *gate, *up, *down;            // routed data
    const uint8_t *gate_s, *up_s, *down_s;      // MXFP4 scales, Q4K parameters (else null)
    const uint16_t *sh_gate, *sh_up, *sh_down;  // bf16 shared (null if none)
    const void* x;                              // [T][H] act dtype
    const int32_t *offsets, *sorted_pair, *active;
    void* h;           // [T*k][F] SwiGLU output of routed pairs (sorted rows)
    void* sh_h;        // [T][Fs] SwiGLU output of the shared expert
    void* expert_out;  // [T*k][H] act dtype
    void* shared_out;  // [T][H] act dtype (null = skip the shared expert)
    int32_t* plan;     // grouped GEMM chunk list (grouped_plan_bytes of workspace)
    // MXFP4 routed experts on fp8 operands (grouped GEMM): the routed experts
    // read x and h as MXFP8-E4M3; h then holds [T*k][F] E4M3 codes.
    int mx8 = 0;
    const uint8_t* xq = nullptr;   // [T][H] E4M3 codes of x
    const uint8_t* xsc = nullptr;  // [T][H/32] E8M0 scales of x
    uint8_t* hsc = nullptr;        // [T*k][F/32] E8M0 scales of h
};

// Routed weight formats (the ABI's ds4moe_wfmt values).
constexpr int WFMT_Q2K = 1, WFMT_MX = 2, WFMT_BF16 = 3, WFMT_Q4K = 4;

// Per-expert byte strides of a routed [rows][K] matrix: data (Q2K blocks, or
// the 4-bit code array of MXFP4 and Q4K) and the second array (MXFP4 E8M0
// scales, Q4K 20-byte super-block parameters).
__host__ __device__ inline size_t expert_data_stride(int wfmt, int rows, int K) {
    return wfmt == WFMT_Q2K ? (size_t)rows * K / 256 * 84 : (size_t)rows * K / 2;
}
__host__ __device__ inline size_t expert_scale_stride(int wfmt, int rows, int K) {
    return wfmt == WFMT_Q4K ? (size_t)rows * K / 256 * 20 : (size_t)rows * K / 32;
}

// Router projection logits[T][E] = x[T][H] . W_r[E][H]^T (bf16 W_r; x bf16,
// or fp32 when f32x), fp32 results.
hipError_t launch_router_logits(const void* x, bool f32x, const uint16_t* w, int T, int H, int E, float* logits,
                                hipStream_t s);
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_pos, int32_t* active, hipStream_t s);
size_t permute_lds_bytes(int E, int T);
// The same permutation for many tokens, spread over token blocks (needs
// permute_scratch_bytes of device scratch).
size_t permute_scratch_bytes(int E, int T);
hipError_t launch_permute_blocked(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* sorted_pair,
                                  int32_t* pair_pos, int32_t* active, int32_t* scratch, hipStream_t s);

// MXFP8-E4M3 quantization of n bf16 values (n % 32 == 0): codes q[n], E8M0
// scales[n/32] (not part of any stage's timing).
hipError_t launch_quantize_mx8(const uint16_t* x, int64_t n, uint8_t* q, uint8_t* scales, hipStream_t s);

hipError_t launch_dequantize(int wfmt, const uint8_t* data, const uint8_t* scales, int64_t n, float* f32,
                             uint16_t* bf16, hipStream_t s);

// fp32 mode: exact fp32 weights, fp32 FMA, any token count.
hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s);

// bf16 path, GEMV kernels (decode): Q2K or MXFP4 routed experts with few
// tokens each, and the bf16 shared expert.
hipError_t launch_ffn_gemv_bf16(const FfnArgs& a, bool routed, bool shared, hipStream_t s);

// bf16 path, grouped GEMM on the matrix cores (prefill).
hipError_t launch_ffn_grouped_bf16(const FfnArgs& a, bool routed, bool shared, hipStream_t s);
size_t grouped_plan_bytes(int E, int T, int k, bool shared);
// The same in two steps: the plan lists the chunks of the active experts (and
// the shared expert's first, when `shared`); the GEMM launches run them.
hipError_t launch_grouped_plan(const FfnArgs& a, bool routed, bool shared, hipStream_t s);
hipError_t launch_grouped_gemm(const FfnArgs& a, bool routed, bool shared, hipStream_t s);
bool grouped_supported(const FfnArgs& a);   // token-row sources below 4 GiB
bool grouped_supports_q4k();

// bf16 path, batch-1 decode (T == 1): the whole layer (route, gate/up +
// SwiGLU, down, weighted combine with the shared expert) in two launches.
struct T1Params {
    int wfmt, H, F, Fs, E, k;
    const float* logits;                        // [E]
    const uint16_t* x;                          // [H] bf16
    const uint8_t *gate, *up, *down;
    const uint8_t *gate_s, *up_s, *down_s;
    const uint16_t *sh_gate, *sh_up, *sh_down;  // null when Fs == 0
    uint16_t* h;                                // [k][F] bf16 scratch
    uint16_t* sh_h;                             // [Fs] bf16 scratch
    uint16_t* y;                                // [H] bf16
    int32_t* sel;                               // [k] scratch: the routing, up launch -> down launch
    float* selw;                                // [k] scratch
};
bool t1_supported(int wfmt, int H, int F, int Fs, int E, int k);
hipError_t launch_layer_t1(const T1Params& p, hipStream_t s);

hipError_t launch_combine(int act_bf16, int T, int H, int k, const void* expert_out, const int32_t* pair_pos,
                          const float* topk_w, const void* shared_out, void* y, hipStream_t s);

}  // namespace ds4
