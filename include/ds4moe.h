/*
 * ds4moe: one routed-MoE layer over low-bit experts, on one AMD Instinct
 * MI355X (gfx950).  C ABI.
 *
 * The layer: a router picks k of E experts per token; each picked expert is a
 * SwiGLU FFN whose gate/up/down weights are stored in a low-bit format
 * (Q2K-style 2-bit super-blocks, or OCP MXFP4); one always-on shared expert
 * with bf16 weights is added; the output is the weighted sum.  The pages this
 * follows say that only the routed experts are quantized while the shared
 * expert, the projections and routing stay at original precision, that the
 * 2-bit experts use Q2_K super-blocks and that an MXFP4 variant keeps the
 * published expert weights (hysenlabs "DwarfStar実地分析", section
 * "GGUFの対応範囲は意図的に狭い"; README mirror "DS4 分布式Shell客户端",
 * section "模型下载"), and that decode is bound by memory bandwidth
 * ("284B MoEを128GBノートPCに詰め込む", section
 * "プリフィル790 t/sが暴く真のボトルネック").
 *
 * Conventions for every call:
 *   - Pointers are device pointers on the current HIP device unless stated;
 *     every pointer must be 16-byte aligned.  The caller allocates and owns
 *     all memory; the library never allocates, frees or keeps a pointer past
 *     the call (ds4moe_forward_noalloc's fixed per-device array aside).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue work and return without synchronising.
 *   - Arguments are validated on the host before anything is enqueued: a
 *     negative status means nothing was launched.  After a launch the HIP
 *     launch status is checked and mapped to DS4MOE_E_HIP.  No call prints,
 *     throws or aborts; ds4moe_last_error() gives a thread-local detail.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics anywhere).  Calls are reentrant; calls that
 *     share output or workspace buffers must be ordered by the caller.
 *
 * Shapes (ds4moe_config):
 *   1 <= top_k <= min(n_experts, 64), n_experts <= 1024,
 *   hidden % 256 == 0, ffn % 128 == 0, shared_ffn % 128 == 0 (0 = none),
 *   hidden, ffn, shared_ffn <= 32768, 1 <= T <= 2^20 and T * top_k < 2^31.
 * These are narrower than the layer's definition, which allows any
 * 1 <= k <= E and, for Q2K, any contraction length that is a multiple of 16
 * with rows * K a multiple of 256: top_k above 64, a hidden width that is not
 * a whole number of 256-weight super-blocks, or an ffn width that is not a
 * whole number of 128-column tiles return DS4MOE_E_SHAPE.  Every
 * configuration named in the workloads (hidden 7168 or 256, ffn 2048 or 128,
 * 256 or 8 experts, top-8 or top-2) lies inside them.
 * Routed matrices: gate and up are [E][ffn][hidden], down is [E][hidden][ffn]
 * (rows x contraction dim, row-major, experts back to back).
 *   Q2K:   84-byte blocks over each expert's flat row-major weights; block b
 *          covers flat weights 256b..256b+255: bytes 0..15 scale s_j (low
 *          nibble) and min m_j (high nibble) of group j (16 weights), bytes
 *          16..79 2-bit codes (code i at byte 16+i/4, bits 2*(i%4)), bytes
 *          80..81 d and 82..83 dmin as little-endian fp16;
 *          weight = d*s_j*q - dmin*m_j.  *_scales pointers must be NULL.
 *   MXFP4: codes [E][rows][K/2] (element c in byte c/2, low nibble when c is
 *          even; E2M1 nibble), scales [E][rows][K/32] E8M0 bytes
 *          (2^(s-127)); weight = E2M1 * scale.  Scale byte 255 (NaN) is an
 *          undefined input.
 *   Q4K:   the 4-bit analogue of the Q2K block, 148 bytes per 256 weights in
 *          two arrays: codes [E][rows][K/2] (element c in byte c/2, low
 *          nibble when c is even; q = 0..15), and in the *_scales pointers
 *          [E][rows][K/256] 20-byte records: bytes 0..15 s_j | m_j << 4 of
 *          group j (16 weights), bytes 16..17 d and 18..19 dmin as
 *          little-endian fp16; weight = d*s_j*q - dmin*m_j.  Requires
 *          ffn % 256 == 0 (ds4moe_dequantize takes records at any 4-byte
 *          alignment).  The pages
 *          name 4-bit expert files (a 2-bit stack whose last six layers'
 *          experts are 4-bit, and a 4-bit model: README mirror
 *          "DS4 分布式Shell客户端", section "模型下载") but no layout; this
 *          one is the library's.
 * Shared expert (bf16 bit patterns): sh_gate, sh_up [shared_ffn][hidden],
 * sh_down [hidden][shared_ffn]; all NULL when shared_ffn == 0.
 *
 * Precision modes (act_dtype):
 *   DS4MOE_DT_F32  "fp32 mode": x, y, stage outputs fp32; weights used as
 *                  their exact fp32 values; fp32 arithmetic throughout.
 *   DS4MOE_DT_BF16 "bf16 path": x, y, stage outputs bf16 (round to nearest
 *                  even); fp32 accumulation; the SwiGLU intermediate h is
 *                  rounded to bf16 before the down projection.
 * Matrix-core operands (mma_dtype), for MXFP4 routed experts in the bf16
 * path:
 *   DS4MOE_DT_BF16     weights decoded exactly to bf16, bf16 x and h.
 *   DS4MOE_DT_FP8_E4M3 the routed experts read x and h as MXFP8-E4M3 (see
 *                  ds4moe_quantize_mxfp8; h is quantized from its fp32 value)
 *                  and run on gfx950's scaled matrix instructions with the
 *                  stored E2M1 codes and E8M0 scales as they are.  Every
 *                  routed expert then uses the grouped GEMM (algo AUTO or
 *                  GROUPED; GEMV, Q2K or fp32 mode: DS4MOE_E_UNSUPPORTED).
 *                  The shared expert stays on bf16 operands.
 */
#ifndef DS4MOE_H
#define DS4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DS4MOE_OK = 0,
    DS4MOE_E_ARG = -1,          /* NULL pointer, bad enum value              */
    DS4MOE_E_SHAPE = -2,        /* sizes outside the limits above            */
    DS4MOE_E_ALIGN = -3,        /* a pointer not 16-byte aligned             */
    DS4MOE_E_UNSUPPORTED = -4,  /* valid but not implemented combination     */
    DS4MOE_E_WORKSPACE = -5,    /* workspace NULL or smaller than required   */
    DS4MOE_E_HIP = -6           /* a HIP launch or runtime call failed       */
} ds4moe_status;

typedef enum { DS4MOE_WFMT_Q2K = 1, DS4MOE_WFMT_MXFP4 = 2, DS4MOE_WFMT_BF16 = 3, DS4MOE_WFMT_Q4K = 4 } ds4moe_wfmt;
typedef enum { DS4MOE_DT_F32 = 0, DS4MOE_DT_BF16 = 1, DS4MOE_DT_FP8_E4M3 = 2 } ds4moe_dtype;
/* Expert-FFN kernel choice.  GEMV streams each touched expert's weights once
 * per small token group (decode); GROUPED runs a dequantize-into-LDS grouped
 * GEMM on the matrix cores (prefill).  AUTO picks per call from the token
 * count T: the batch-1 path at T = 1 where supported, GEMV up to 8 tokens,
 * GROUPED above.  fp32 mode always uses GEMV (GROUPED is
 * DS4MOE_E_UNSUPPORTED). */
typedef enum { DS4MOE_ALGO_AUTO = 0, DS4MOE_ALGO_GEMV = 1, DS4MOE_ALGO_GROUPED = 2 } ds4moe_algo;

typedef struct {
    int32_t hidden;      /* H: model width                                   */
    int32_t ffn;         /* F: routed expert FFN width                       */
    int32_t n_experts;   /* E                                                */
    int32_t top_k;       /* k                                                */
    int32_t shared_ffn;  /* Fs: shared expert FFN width, 0 = no shared expert */
    int32_t wfmt;        /* ds4moe_wfmt of the routed weights (Q2K or MXFP4) */
    int32_t act_dtype;   /* ds4moe_dtype: F32 or BF16                        */
    int32_t mma_dtype;   /* MXFP4 matrix-core operands: BF16 (default) or FP8_E4M3 */
    int32_t algo;        /* ds4moe_algo                                      */
} ds4moe_config;

typedef struct {
    const void *gate, *up, *down;                      /* routed, in cfg.wfmt   */
    const void *gate_scales, *up_scales, *down_scales; /* MXFP4 E8M0, else NULL */
    const void *sh_gate, *sh_up, *sh_down;             /* bf16, NULL if none    */
} ds4moe_weights;

/* Router projection: logits[t][e] = sum_h router_w[e][h] * x[t][h] for every
 * token t < T and expert e < n_experts, the step that feeds ds4moe_route.
 * The pages keep the router at original precision while only the routed
 * experts are quantized (hysenlabs page, section above); this library reads
 * that as bf16 router weights with fp32 accumulation.  router_w: bf16 bit
 * patterns [n_experts][hidden], row-major; x: [T][hidden] in act_dtype (bf16,
 * or fp32 in fp32 mode); logits: fp32 [T][n_experts], every element written.
 * bf16 x bf16 products are exact in fp32; the order of the fp32 additions is
 * the library's (fixed for a given T, so results are reproducible), within
 * (hidden - 1) * 2^-24 * sum_h |router_w[e][h] * x[t][h]| of the exact sum.
 * Only the x, router_w and logits pointers are read; other config fields
 * must still be valid. */
int ds4moe_router_logits(const ds4moe_config* cfg, int32_t T, const void* x, const void* router_w,
                         float* logits, void* stream);

/* Router top-k.  For each token t: keep the k largest of logits[t][0..E) with
 * ties to the lower expert index (-0 == +0), slot j = j-th kept expert in
 * (logit descending, index ascending) order; topk_w[t][j] = softmax over the
 * kept logits (= softmax over all E, select, renormalise).  The pages keep
 * routing at original precision (hysenlabs page, section above); the rule is
 * this library's reading.  logits: fp32 [T][E]; topk_idx: int32 [T][k];
 * topk_w: fp32 [T][k].  NaN logits are undefined input. */
int ds4moe_route(const ds4moe_config* cfg, int32_t T, const float* logits,
                 int32_t* topk_idx, float* topk_w, void* stream);

/* Token-to-expert permutation: histogram of topk_idx over E experts,
 * exclusive prefix sum, stable scatter.  Pair id p = t*k + j.  The pages
 * give no interface for this step (their engine's expert kernels are not
 * shown); it is the grouping of (token, expert) pairs by expert that batched
 * expert work on matrix instructions needs (hysenlabs "DwarfStar実地分析",
 * section "GGUFの対応範囲は意図的に狭い"), with the order fixed by this
 * library so the result is unique and checkable.
 *   expert_offsets int32 [E+1]: offsets[e] = #pairs routed to experts < e
 *   sorted_pair    int32 [T*k]: pairs by expert ascending, token ascending
 *   pair_pos       int32 [T*k]: inverse, pair_pos[sorted_pair[r]] = r
 *   active         int32 [E+1]: active[0] = n experts with pairs, then their
 *                               ids ascending (unused tail left as is)
 * topk_idx must hold valid ids, distinct within a token (as route makes). */
int ds4moe_permute(const ds4moe_config* cfg, int32_t T, const int32_t* topk_idx,
                   int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                   int32_t* active, void* stream);

/* Expert FFNs.  For every sorted row r (pair p = sorted_pair[r], token
 * t = p / k, expert e): expert_out[r] = W_d^e (silu(W_g^e x_t) * W_u^e x_t),
 * and when the layer has a shared expert, shared_out[t] = the same SwiGLU FFN
 * with the bf16 shared weights, for every token.  The routed up/gate/down
 * matrices are the low-bit tensors and the shared expert stays at original
 * precision (hysenlabs "DwarfStar実地分析", section
 * "GGUFの対応範囲は意図的に狭い"); decode streams these weights and is bound
 * by memory bandwidth ("284B MoEを128GBノートPCに詰め込む", section
 * "プリフィル790 t/sが暴く真のボトルネック").  The SwiGLU activation (gate
 * through silu, no clamp) is this library's reading: the pages do not state
 * the expert's activation.  x: [T][H] in act_dtype;
 * expert_out: [T*k][H] act_dtype; shared_out: [T][H] act_dtype, or NULL
 * (then the shared expert is skipped).  workspace: device scratch of at least
 * ds4moe_workspace_bytes(cfg, T) bytes (contents undefined on return). */
int ds4moe_expert_ffn(const ds4moe_config* cfg, const ds4moe_weights* w, int32_t T,
                      const void* x, const int32_t* expert_offsets, const int32_t* sorted_pair,
                      const int32_t* active, void* expert_out, void* shared_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Weighted combine: y[t] = shared_out[t] + sum_j topk_w[t][j] *
 * expert_out[pair_pos[t*k+j]], summed in fp32 in slot order j = 0..k-1
 * (gather form of the scatter-combine; no atomics).  The pages do not spell
 * this step out; the shared expert added with weight 1 to the routed sum is
 * this library's reading of an always-on shared expert that the pages'
 * tensor-parallel split keeps whole on every machine while the routed experts
 * are split in halves (hysenlabs "DwarfStar実地分析", section
 * "RDMAとCUDAテンソル並列は分割の仕方が違う").  shared_out may be NULL
 * (treated as zero).  A pair_pos entry outside [0, T*k) adds nothing (its
 * slot is skipped, so corrupt input reads no row outside expert_out).
 * expert_out, shared_out, y in act_dtype. */
int ds4moe_combine(const ds4moe_config* cfg, int32_t T, const void* expert_out,
                   const int32_t* pair_pos, const float* topk_w, const void* shared_out,
                   void* y, void* stream);

/* The whole layer: route, permute, expert FFNs (+ shared), combine, using
 * workspace for every intermediate.  x [T][H] and y [T][H] in act_dtype,
 * logits fp32 [T][E].  Kernels may be fused internally; the result is the
 * same layer.  This is the routed-MoE layer of the pages' model: a shared
 * expert plus k routed low-bit experts per token (hysenlabs "DwarfStar実地分析",
 * section "GGUFの対応範囲は意図的に狭い"), run for one decode token or a
 * prefill chunk (Qiita "複数 Mac で 1 つのモデルを動かす", section
 * "3. prefill", 4096-token chunks). */
int ds4moe_forward(const ds4moe_config* cfg, const ds4moe_weights* w, int32_t T,
                   const void* x, const float* logits, void* y,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ds4moe_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same launches and results as
 * ds4moe_forward, with the workspace in a fixed device array inside the
 * library: ds4moe_forward_noalloc_max_bytes() bytes (64 MiB) per device,
 * held from the first call on that device until the process ends.  x, y and
 * the weights are the caller's as for ds4moe_forward; nothing is allocated or
 * freed.  DS4MOE_E_WORKSPACE when ds4moe_workspace_bytes(cfg, T) exceeds that
 * size (for the 7168/2048, 256-expert top-8 layer with a 2048-wide shared
 * expert, T up to about 380 fits).  Every call on one device shares that
 * device's array, which keeps the last call's contents: calls that overlap on
 * one device (other streams, other threads) race and must be ordered by the
 * caller.  The first call on a device looks the array's address up
 * (DS4MOE_E_HIP if that fails). */
int ds4moe_forward_noalloc(const ds4moe_config* cfg, const ds4moe_weights* w, int32_t T,
                           const void* x, const float* logits, void* y, void* stream);
size_t ds4moe_forward_noalloc_max_bytes(void);

/* Workspace bytes that ds4moe_forward and ds4moe_expert_ffn need for up to
 * T_max tokens (0 on an invalid config). */
size_t ds4moe_workspace_bytes(const ds4moe_config* cfg, int32_t T_max);

/* Where ds4moe_forward keeps a stage's result inside its workspace, for
 * inspection (tests): after a forward call with this cfg and T that returned
 * DS4MOE_OK, and once its stream has drained, the workspace bytes
 * [*offset, *offset + *bytes) hold
 *   DS4MOE_WS_TOPK_IDX     int32 [T][k]  the route's expert ids (slot order)
 *   DS4MOE_WS_TOPK_W       fp32 [T][k]   the route's weights
 *   DS4MOE_WS_OFFSETS      int32 [E+1]   the permutation, exactly as
 *   DS4MOE_WS_SORTED_PAIR  int32 [T*k]   ds4moe_permute defines its four
 *   DS4MOE_WS_PAIR_POS     int32 [T*k]   outputs (forward may compute them
 *   DS4MOE_WS_ACTIVE       int32 [E+1]   with a different kernel)
 *   DS4MOE_WS_EXPERT_OUT   act [T*k][H]  routed expert outputs, sorted rows
 *   DS4MOE_WS_SHARED_OUT   act [T][H]    the shared expert's output
 * The batch-1 launch sequence (ds4moe_forward_path 1) keeps none of these
 * except TOPK_IDX and TOPK_W; every other region is then left as it was.
 * Offsets are multiples of 256.  DS4MOE_E_ARG for an unknown region or NULL
 * outputs; the config and T are checked as for ds4moe_forward.  Nothing is
 * enqueued. */
typedef enum {
    DS4MOE_WS_TOPK_IDX = 0, DS4MOE_WS_TOPK_W = 1, DS4MOE_WS_OFFSETS = 2, DS4MOE_WS_SORTED_PAIR = 3,
    DS4MOE_WS_PAIR_POS = 4, DS4MOE_WS_ACTIVE = 5, DS4MOE_WS_EXPERT_OUT = 6, DS4MOE_WS_SHARED_OUT = 7
} ds4moe_ws_region;
int ds4moe_workspace_region(const ds4moe_config* cfg, int32_t T, int32_t region, size_t* offset,
                            size_t* bytes);

/* Test export: decode n weights of a flat weight array in format wfmt (Q2K:
 * n % 256 == 0; MXFP4: n % 32 == 0 with scales = its E8M0 array; BF16:
 * n % 16 == 0) through the same device decode routines the expert kernels
 * use.  out_f32 receives each weight's exact value rounded to fp32, out_bf16
 * that fp32 value rounded to bf16 (nearest even) as bit patterns; either may
 * be NULL (not both). */
int ds4moe_dequantize(int32_t wfmt, const void* data, const void* scales, int64_t n,
                      float* out_f32, uint16_t* out_bf16, void* stream);

/* MXFP8-E4M3 quantization (OCP MX v1.0 block rule, the fp8 operand of the
 * MXFP4 experts): n bf16 values (n % 32 == 0) in blocks of 32 consecutive
 * values; per block the E8M0 scale byte s = floor(log2 amax) - 8 + 127 (8 is
 * E4M3's largest exponent), held at 0 when lower, and 127 for an all-zero
 * block; code j = value j / 2^(s-127) rounded to nearest-even OCP E4M3 (bias
 * 7, max 448), saturating at +-448.  The pages pack 8-bit activations as an
 * E4M3-like f8 (qiita "DwarfStar の TCP パイプライン分散推論を読む", section
 * 9); the block scaling is OCP MX's.  x_bf16 [n] bf16 bit patterns; codes
 * [n] bytes; scales [n/32] bytes (any alignment).  The same rule and device
 * routine quantize x inside ds4moe_forward / ds4moe_expert_ffn when
 * mma_dtype is FP8_E4M3. */
int ds4moe_quantize_mxfp8(const void* x_bf16, int64_t n, uint8_t* codes, uint8_t* scales,
                          void* stream);

/* Kernel stages, for per-stage timing. */
typedef enum {
    DS4MOE_STAGE_ROUTE = 0,     /* router top-k kernel                        */
    DS4MOE_STAGE_PERMUTE = 1,   /* histogram / prefix-sum permutation kernel  */
    DS4MOE_STAGE_FFN_UP = 2,    /* gate/up projections + SwiGLU (routed+shared) */
    DS4MOE_STAGE_FFN_DOWN = 3,  /* down projections (routed + shared)         */
    DS4MOE_STAGE_COMBINE = 4,   /* weighted combine                           */
    DS4MOE_STAGE_ROUTER_PROJ = 5 /* router projection (ds4moe_router_logits)  */
} ds4moe_stage;

/* Instrumentation.  Until cleared, the kernel launches of `stage` made by
 * this thread record start_event when the stage's first launch in a call
 * starts and stop_event when its last launch ends (hipEvent_t handles passed
 * as void*; the caller creates them).  NULL, NULL clears.  Per-stage timing in the spirit of the pages' per-hop telemetry
 * (Qiita "複数 Mac で 1 つのモデルを動かす: DwarfStar の TCP パイプライン分散推論
 * を読む", section "8. RESULT: ACK / 隠れ状態 / logits"). */
int ds4moe_set_stage_events(int stage, void* start_event, void* stop_event);

/* The launch sequence ds4moe_forward takes for this configuration and token
 * count: 1 = batch 1 in two launches (routing fused into the gate/up launch,
 * the weighted combine into the down launch; bf16 path, AUTO, supported
 * shapes); otherwise route, permute, expert FFN and combine launches, with
 * the expert FFNs on the GEMV kernels (0; also fp32 mode) or on the grouped
 * GEMM (2).  Negative status on an invalid configuration. */
int ds4moe_forward_path(const ds4moe_config* cfg, int32_t T);

/* Static description of a status code. */
const char* ds4moe_status_string(int status);

/* Thread-local detail for the last non-OK return on this thread ("" if none). */
const char* ds4moe_last_error(void);

/* Library version string. */
const char* ds4moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DS4MOE_H */
