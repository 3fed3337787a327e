// C-ABI entry points of libds4moe: host-side validation, workspace layout and
// kernel orchestration.  Every check happens before the first launch, so a
// non-OK return means nothing was enqueued.
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "ds4moe.h"
#include "launch.hpp"

namespace ds4 {
thread_local StageEvents g_stage_events[N_STAGES] = {};
thread_local bool g_stage_started[N_STAGES] = {};
// The start event goes with the first launch of a stage in an API call, the
// stop event with every launch (the last one's record stands).
StageEvents stage_events(int stage) {
    StageEvents ev = g_stage_events[stage];
    if (g_stage_started[stage]) ev.start = nullptr;
    g_stage_started[stage] = true;
    return ev;
}
void stage_call_begin() {
    for (int i = 0; i < N_STAGES; ++i) g_stage_started[i] = false;
}
}  // namespace ds4

// Workspace of ds4moe_forward_noalloc (see there).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return DS4MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DS4MOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Token count at or below which AUTO runs the expert FFNs on the GEMV kernels
// (above it, on the grouped GEMM).  Measured on MI355X over 5..32 tokens of
// the 7168/2048, 256-expert top-8 layer: the GEMV kernels lead up to 7 tokens
// under Zipf(1.1) routing (a tie at 8) and up to 16 under uniform routing; with
// the cut at 8 the slower choice costs about 11% at most (uniform routing at
// 10 to 16 tokens).  Splitting one call between both kernels by tokens per
// expert was slower than either alone at every count from 5 up.
constexpr int AUTO_GEMV_MAX_TOKENS = 8;
// Token count from which forward spreads the permutation over token blocks
// (below it one workgroup is quicker than three launches).
constexpr int PERMUTE_BLOCKED_MIN_TOKENS = 256;
// Largest hidden, ffn and shared_ffn (see check_cfg).
constexpr int MAX_WIDTH = 32768;

// Whether a bf16-path call with T tokens runs its expert FFNs on the grouped
// GEMM (else on the GEMV kernels): fp8 operands and GROUPED always, AUTO above
// AUTO_GEMV_MAX_TOKENS while the token-row sources fit its 32-bit offsets.
bool ffn_grouped(const ds4moe_config* c, int32_t T, const ds4::FfnArgs& a) {
    if (c->act_dtype == DS4MOE_DT_F32) return false;
    if (c->wfmt == DS4MOE_WFMT_Q4K && !ds4::grouped_supports_q4k()) return false;
    if (c->mma_dtype == DS4MOE_DT_FP8_E4M3 || c->algo == DS4MOE_ALGO_GROUPED) return true;
    if (c->algo == DS4MOE_ALGO_GEMV) return false;
    return T > AUTO_GEMV_MAX_TOKENS && ds4::grouped_supported(a);
}

int check_cfg(const ds4moe_config* c) {
    if (!c) return fail(DS4MOE_E_ARG, "cfg is NULL");
    if (c->wfmt != DS4MOE_WFMT_Q2K && c->wfmt != DS4MOE_WFMT_MXFP4 && c->wfmt != DS4MOE_WFMT_Q4K) {
        if (c->wfmt == DS4MOE_WFMT_BF16) return fail(DS4MOE_E_UNSUPPORTED, "bf16 routed experts are not supported");
        return fail(DS4MOE_E_ARG, "wfmt %d is not a routed weight format", c->wfmt);
    }
    if (c->act_dtype != DS4MOE_DT_F32 && c->act_dtype != DS4MOE_DT_BF16) {
        if (c->act_dtype == DS4MOE_DT_FP8_E4M3) return fail(DS4MOE_E_UNSUPPORTED, "fp8 activations in/out");
        return fail(DS4MOE_E_ARG, "act_dtype %d", c->act_dtype);
    }
    if (c->mma_dtype != DS4MOE_DT_BF16 && c->mma_dtype != DS4MOE_DT_FP8_E4M3 && c->mma_dtype != DS4MOE_DT_F32)
        return fail(DS4MOE_E_ARG, "mma_dtype %d", c->mma_dtype);
    if (c->mma_dtype == DS4MOE_DT_FP8_E4M3) {
        if (c->wfmt != DS4MOE_WFMT_MXFP4)
            return fail(DS4MOE_E_UNSUPPORTED, "fp8 matrix-core operands need MXFP4 routed experts");
        if (c->act_dtype != DS4MOE_DT_BF16)
            return fail(DS4MOE_E_UNSUPPORTED, "fp8 matrix-core operands need bf16 activations");
        if (c->algo == DS4MOE_ALGO_GEMV)
            return fail(DS4MOE_E_UNSUPPORTED, "fp8 matrix-core operands run on the grouped GEMM only");
    }
    if (c->algo < DS4MOE_ALGO_AUTO || c->algo > DS4MOE_ALGO_GROUPED) return fail(DS4MOE_E_ARG, "algo %d", c->algo);
    if (c->n_experts < 1 || c->n_experts > 1024) return fail(DS4MOE_E_SHAPE, "n_experts %d not in [1, 1024]", c->n_experts);
    const int kmax = c->n_experts < 64 ? c->n_experts : 64;
    if (c->top_k < 1 || c->top_k > kmax) return fail(DS4MOE_E_SHAPE, "top_k %d not in [1, %d]", c->top_k, kmax);
    // Width limits: every kernel's LDS staging of one token's activations
    // (the fp32-mode kernels hold a whole fp32 row, 4 * 32768 = 128 KiB, of
    // the 160 KiB a workgroup may use) fits at these sizes, so a call never
    // fails at a launch after earlier launches were enqueued.
    if (c->hidden < 256 || c->hidden % 256 || c->hidden > MAX_WIDTH)
        return fail(DS4MOE_E_SHAPE, "hidden %d must be a multiple of 256 in [256, %d]", c->hidden, MAX_WIDTH);
    if (c->ffn < 128 || c->ffn % 128 || c->ffn > MAX_WIDTH)
        return fail(DS4MOE_E_SHAPE, "ffn %d must be a multiple of 128 in [128, %d]", c->ffn, MAX_WIDTH);
    if (c->shared_ffn < 0 || c->shared_ffn % 128 || c->shared_ffn > MAX_WIDTH)
        return fail(DS4MOE_E_SHAPE, "shared_ffn %d must be 0 or a multiple of 128 up to %d", c->shared_ffn,
                    MAX_WIDTH);
    if (c->act_dtype == DS4MOE_DT_F32 && c->algo == DS4MOE_ALGO_GROUPED)
        return fail(DS4MOE_E_UNSUPPORTED, "fp32 mode runs the GEMV kernels only");
    if (c->wfmt == DS4MOE_WFMT_Q4K && c->ffn % 256)
        return fail(DS4MOE_E_SHAPE, "Q4K rows are whole 256-weight super-blocks: ffn %d must be a multiple of 256",
                    c->ffn);
    return DS4MOE_OK;
}

int check_T(const ds4moe_config* c, int32_t T) {
    if (T < 1 || T > (1 << 20)) return fail(DS4MOE_E_SHAPE, "T %d not in [1, 2^20]", T);
    if ((int64_t)T * c->top_k >= (int64_t)INT_MAX) return fail(DS4MOE_E_SHAPE, "T * top_k overflows int32");
    return DS4MOE_OK;
}

int check_weights(const ds4moe_config* c, const ds4moe_weights* w) {
    if (!w) return fail(DS4MOE_E_ARG, "weights is NULL");
    if (!w->gate || !w->up || !w->down) return fail(DS4MOE_E_ARG, "routed weight pointer is NULL");
    if (c->wfmt == DS4MOE_WFMT_MXFP4 || c->wfmt == DS4MOE_WFMT_Q4K) {
        if (!w->gate_scales || !w->up_scales || !w->down_scales)
            return fail(DS4MOE_E_ARG, "%s are NULL", c->wfmt == DS4MOE_WFMT_MXFP4 ? "MXFP4 scales" : "Q4K parameters");
    } else if (w->gate_scales || w->up_scales || w->down_scales) {
        return fail(DS4MOE_E_ARG, "scales must be NULL for Q2K");
    }
    if (c->shared_ffn > 0) {
        if (!w->sh_gate || !w->sh_up || !w->sh_down) return fail(DS4MOE_E_ARG, "shared weight pointer is NULL");
    } else if (w->sh_gate || w->sh_up || w->sh_down) {
        return fail(DS4MOE_E_ARG, "shared weights given but shared_ffn == 0");
    }
    const void* ps[] = {w->gate, w->up, w->down, w->gate_scales, w->up_scales, w->down_scales,
                        w->sh_gate, w->sh_up, w->sh_down};
    for (const void* p : ps)
        if (p && !aligned16(p)) return fail(DS4MOE_E_ALIGN, "weight pointer %p not 16-byte aligned", p);
    return DS4MOE_OK;
}

#define REQ_PTR(p)                                                                     \
    do {                                                                               \
        if (!(p)) return fail(DS4MOE_E_ARG, "%s is NULL", #p);                         \
        if (!aligned16(p)) return fail(DS4MOE_E_ALIGN, "%s not 16-byte aligned", #p);  \
    } while (0)

#define OPT_PTR(p)                                                                     \
    do {                                                                               \
        if ((p) && !aligned16(p)) return fail(DS4MOE_E_ALIGN, "%s not 16-byte aligned", #p); \
    } while (0)

#define TRY(expr)                     \
    do {                              \
        const int st_ = (expr);       \
        if (st_ != DS4MOE_OK) return st_; \
    } while (0)

struct WsLayout {
    size_t idx, w, off, sp, pp, act, h, shh, eo, so, plan, perm, xq, xsc, hsc, total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const ds4moe_config* c, int32_t T) {
    const size_t P = (size_t)T * c->top_k;
    const size_t E1 = (size_t)c->n_experts + 1;
    const size_t eb = c->act_dtype == DS4MOE_DT_F32 ? 4 : 2;
    WsLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = align256(off);
        off = o + bytes;
        return o;
    };
    L.idx = take(P * 4);
    L.w = take(P * 4);
    L.off = take(E1 * 4);
    L.sp = take(P * 4);
    L.pp = take(P * 4);
    L.act = take(E1 * 4);
    L.h = take(P * c->ffn * eb);
    L.shh = take((size_t)T * c->shared_ffn * eb);
    L.eo = take(P * c->hidden * eb);
    L.so = take((size_t)T * c->hidden * eb);
    L.plan = take(ds4::grouped_plan_bytes(c->n_experts, T, c->top_k, c->shared_ffn > 0));
    L.perm = take(ds4::permute_scratch_bytes(c->n_experts, T));
    const bool mx8 = c->mma_dtype == DS4MOE_DT_FP8_E4M3;   // h above then holds E4M3 codes
    L.xq = take(mx8 ? (size_t)T * c->hidden : 0);
    L.xsc = take(mx8 ? (size_t)T * c->hidden / 32 : 0);
    L.hsc = take(mx8 ? P * c->ffn / 32 : 0);
    L.total = align256(off);
    return L;
}

int run_ffn(const ds4moe_config* c, const ds4moe_weights* w, int32_t T, const void* x, const int32_t* offsets,
            const int32_t* sorted_pair, const int32_t* active, void* eo, void* so, void* ws, hipStream_t s) {
    const WsLayout L = ws_layout(c, T);
    ds4::FfnArgs a;
    a.H = c->hidden;
    a.F = c->ffn;
    a.Fs = so ? c->shared_ffn : 0;
    a.E = c->n_experts;
    a.k = c->top_k;
    a.T = T;
    a.wfmt = c->wfmt;
    a.gate = static_cast<const uint8_t*>(w->gate);
    a.up = static_cast<const uint8_t*>(w->up);
    a.down = static_cast<const uint8_t*>(w->down);
    a.gate_s = static_cast<const uint8_t*>(w->gate_scales);
    a.up_s = static_cast<const uint8_t*>(w->up_scales);
    a.down_s = static_cast<const uint8_t*>(w->down_scales);
    a.sh_gate = static_cast<const uint16_t*>(w->sh_gate);
    a.sh_up = static_cast<const uint16_t*>(w->sh_up);
    a.sh_down = static_cast<const uint16_t*>(w->sh_down);
    a.x = x;
    a.offsets = offsets;
    a.sorted_pair = sorted_pair;
    a.active = active;
    a.h = static_cast<uint8_t*>(ws) + L.h;
    a.sh_h = static_cast<uint8_t*>(ws) + L.shh;
    a.expert_out = eo;
    a.shared_out = so;
    a.plan = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + L.plan);
    const bool shared = so != nullptr && c->shared_ffn > 0;
    if (c->act_dtype == DS4MOE_DT_F32) return hip_status(ds4::launch_ffn_f32(a, s), "expert FFN (fp32)");
    if (c->mma_dtype == DS4MOE_DT_FP8_E4M3) {
        // every routed expert on the scaled matrix instructions, x quantized once
        if (!ds4::grouped_supported(a))
            return fail(DS4MOE_E_UNSUPPORTED, "grouped GEMM: x, h and the shared h must each be below 4 GiB");
        uint8_t* xq = static_cast<uint8_t*>(ws) + L.xq;
        uint8_t* xsc = static_cast<uint8_t*>(ws) + L.xsc;
        a.mx8 = 1;
        a.xq = xq;
        a.xsc = xsc;
        a.hsc = static_cast<uint8_t*>(ws) + L.hsc;
        // (outside the stage timings, which cover the projection kernels)
        hipError_t e = ds4::launch_quantize_mx8(static_cast<const uint16_t*>(x), (int64_t)T * c->hidden, xq, xsc, s);
        if (e != hipSuccess) return hip_status(e, "expert FFN (MXFP8 x)");
        return hip_status(ds4::launch_ffn_grouped_bf16(a, true, shared, s), "expert FFN (grouped, fp8 operands)");
    }
    if (c->algo == DS4MOE_ALGO_GROUPED && c->wfmt == DS4MOE_WFMT_Q4K && !ds4::grouped_supports_q4k())
        return fail(DS4MOE_E_UNSUPPORTED, "Q4K experts do not run on the grouped GEMM");
    if (c->algo == DS4MOE_ALGO_GROUPED && !ds4::grouped_supported(a))
        return fail(DS4MOE_E_UNSUPPORTED, "grouped GEMM: x, h and the shared h must each be below 4 GiB");
    if (ffn_grouped(c, T, a)) return hip_status(ds4::launch_ffn_grouped_bf16(a, true, shared, s), "expert FFN (grouped)");
    return hip_status(ds4::launch_ffn_gemv_bf16(a, true, shared, s), "expert FFN (GEMV)");
}

// ---- allocation-free forward ----------------------------------------------------
// ds4moe_forward_noalloc keeps forward's workspace in the file-scope device
// array `scratch` (above).  Each device the library runs on holds its own copy
// (at its own address) until the process ends.  Host code never passes the
// array's name to a kernel or a copy: it uses the device address
// hipGetSymbolAddress returns, looked up once per device.
constexpr int MAX_DEVICES = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's address of `scratch`, or null with the error set.
void* scratch_for_current_device(int* status) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *status = hip_status(e, "forward_noalloc: hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= MAX_DEVICES) {
        *status = fail(DS4MOE_E_UNSUPPORTED, "forward_noalloc: device %d beyond %d", dev, MAX_DEVICES);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *status = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "forward_noalloc: hipGetSymbolAddress");
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    *status = DS4MOE_OK;
    return g_scratch_ptr[dev];
}

bool batch1_path(const ds4moe_config* cfg, int32_t T) {
    return T == 1 && cfg->act_dtype == DS4MOE_DT_BF16 && cfg->mma_dtype != DS4MOE_DT_FP8_E4M3 &&
           cfg->algo == DS4MOE_ALGO_AUTO &&
           ds4::t1_supported(cfg->wfmt, cfg->hidden, cfg->ffn, cfg->shared_ffn, cfg->n_experts, cfg->top_k);
}

}  // namespace

extern "C" {

int ds4moe_forward_path(const ds4moe_config* cfg, int32_t T) {
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    if (batch1_path(cfg, T)) return 1;
    ds4::FfnArgs a{};
    a.H = cfg->hidden;
    a.F = cfg->ffn;
    a.Fs = cfg->shared_ffn;
    a.k = cfg->top_k;
    a.T = T;
    return ffn_grouped(cfg, T, a) ? 2 : 0;
}

const char* ds4moe_version(void) { return "ds4moe 0.1 (gfx950)"; }

const char* ds4moe_status_string(int status) {
    switch (status) {
        case DS4MOE_OK: return "ok";
        case DS4MOE_E_ARG: return "invalid argument";
        case DS4MOE_E_SHAPE: return "shape out of range";
        case DS4MOE_E_ALIGN: return "pointer not 16-byte aligned";
        case DS4MOE_E_UNSUPPORTED: return "unsupported combination";
        case DS4MOE_E_WORKSPACE: return "workspace missing or too small";
        case DS4MOE_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* ds4moe_last_error(void) { return g_last_error.c_str(); }

int ds4moe_set_stage_events(int stage, void* start_event, void* stop_event) {
    if (stage < 0 || stage >= ds4::N_STAGES) return fail(DS4MOE_E_ARG, "stage %d", stage);
    ds4::g_stage_events[stage].start = static_cast<hipEvent_t>(start_event);
    ds4::g_stage_events[stage].stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

size_t ds4moe_workspace_bytes(const ds4moe_config* cfg, int32_t T_max) {
    if (check_cfg(cfg) != DS4MOE_OK || check_T(cfg, T_max) != DS4MOE_OK) return 0;
    return ws_layout(cfg, T_max).total;
}

int ds4moe_workspace_region(const ds4moe_config* cfg, int32_t T, int32_t region, size_t* offset, size_t* bytes) {
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    if (!offset || !bytes) return fail(DS4MOE_E_ARG, "offset or bytes is NULL");
    const WsLayout L = ws_layout(cfg, T);
    const size_t P = (size_t)T * cfg->top_k, E1 = (size_t)cfg->n_experts + 1;
    const size_t eb = cfg->act_dtype == DS4MOE_DT_F32 ? 4 : 2;
    switch (region) {
        case DS4MOE_WS_TOPK_IDX: *offset = L.idx; *bytes = P * 4; break;
        case DS4MOE_WS_TOPK_W: *offset = L.w; *bytes = P * 4; break;
        case DS4MOE_WS_OFFSETS: *offset = L.off; *bytes = E1 * 4; break;
        case DS4MOE_WS_SORTED_PAIR: *offset = L.sp; *bytes = P * 4; break;
        case DS4MOE_WS_PAIR_POS: *offset = L.pp; *bytes = P * 4; break;
        case DS4MOE_WS_ACTIVE: *offset = L.act; *bytes = E1 * 4; break;
        case DS4MOE_WS_EXPERT_OUT: *offset = L.eo; *bytes = P * cfg->hidden * eb; break;
        case DS4MOE_WS_SHARED_OUT: *offset = L.so; *bytes = (size_t)T * cfg->hidden * eb; break;
        default: return fail(DS4MOE_E_ARG, "workspace region %d", region);
    }
    return ok();
}

int ds4moe_router_logits(const ds4moe_config* cfg, int32_t T, const void* x, const void* router_w, float* logits,
                         void* stream) {
    ds4::stage_call_begin();
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    REQ_PTR(x);
    REQ_PTR(router_w);
    REQ_PTR(logits);
    return hip_status(ds4::launch_router_logits(x, cfg->act_dtype == DS4MOE_DT_F32,
                                                static_cast<const uint16_t*>(router_w), T, cfg->hidden,
                                                cfg->n_experts, logits, static_cast<hipStream_t>(stream)),
                      "router_logits");
}

int ds4moe_route(const ds4moe_config* cfg, int32_t T, const float* logits, int32_t* topk_idx, float* topk_w,
                 void* stream) {
    ds4::stage_call_begin();
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    REQ_PTR(logits);
    REQ_PTR(topk_idx);
    REQ_PTR(topk_w);
    return hip_status(ds4::launch_route(logits, T, cfg->n_experts, cfg->top_k, topk_idx, topk_w,
                                        static_cast<hipStream_t>(stream)),
                      "route");
}

int ds4moe_permute(const ds4moe_config* cfg, int32_t T, const int32_t* topk_idx, int32_t* expert_offsets,
                   int32_t* sorted_pair, int32_t* pair_pos, int32_t* active, void* stream) {
    ds4::stage_call_begin();
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    REQ_PTR(topk_idx);
    REQ_PTR(expert_offsets);
    REQ_PTR(sorted_pair);
    REQ_PTR(pair_pos);
    REQ_PTR(active);
    return hip_status(ds4::launch_permute(topk_idx, T, cfg->n_experts, cfg->top_k, expert_offsets, sorted_pair,
                                          pair_pos, active, static_cast<hipStream_t>(stream)),
                      "permute");
}

int ds4moe_expert_ffn(const ds4moe_config* cfg, const ds4moe_weights* w, int32_t T, const void* x,
                      const int32_t* expert_offsets, const int32_t* sorted_pair, const int32_t* active,
                      void* expert_out, void* shared_out, void* workspace, size_t workspace_bytes, void* stream) {
    ds4::stage_call_begin();
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    TRY(check_weights(cfg, w));
    REQ_PTR(x);
    REQ_PTR(expert_offsets);
    REQ_PTR(sorted_pair);
    REQ_PTR(active);
    REQ_PTR(expert_out);
    OPT_PTR(shared_out);
    if (!workspace) return fail(DS4MOE_E_WORKSPACE, "workspace is NULL");
    if (!aligned16(workspace)) return fail(DS4MOE_E_ALIGN, "workspace not 16-byte aligned");
    const size_t need = ws_layout(cfg, T).total;
    if (workspace_bytes < need)
        return fail(DS4MOE_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    void* so = cfg->shared_ffn > 0 ? shared_out : nullptr;
    return run_ffn(cfg, w, T, x, expert_offsets, sorted_pair, active, expert_out, so, workspace,
                   static_cast<hipStream_t>(stream));
}

int ds4moe_combine(const ds4moe_config* cfg, int32_t T, const void* expert_out, const int32_t* pair_pos,
                   const float* topk_w, const void* shared_out, void* y, void* stream) {
    ds4::stage_call_begin();
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    REQ_PTR(expert_out);
    REQ_PTR(pair_pos);
    REQ_PTR(topk_w);
    OPT_PTR(shared_out);
    REQ_PTR(y);
    return hip_status(ds4::launch_combine(cfg->act_dtype == DS4MOE_DT_BF16, T, cfg->hidden, cfg->top_k, expert_out,
                                          pair_pos, topk_w, shared_out, y, static_cast<hipStream_t>(stream)),
                      "combine");
}

int ds4moe_forward(const ds4moe_config* cfg, const ds4moe_weights* w, int32_t T, const void* x, const float* logits,
                   void* y, void* workspace, size_t workspace_bytes, void* stream) {
    ds4::stage_call_begin();
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    TRY(check_weights(cfg, w));
    REQ_PTR(x);
    REQ_PTR(logits);
    REQ_PTR(y);
    if (!workspace) return fail(DS4MOE_E_WORKSPACE, "workspace is NULL");
    if (!aligned16(workspace)) return fail(DS4MOE_E_ALIGN, "workspace not 16-byte aligned");
    const WsLayout L = ws_layout(cfg, T);
    if (workspace_bytes < L.total)
        return fail(DS4MOE_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, L.total);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (batch1_path(cfg, T)) {
        // one token: route, expert FFNs, shared expert and combine in two launches
        ds4::T1Params p;
        p.wfmt = cfg->wfmt;
        p.H = cfg->hidden;
        p.F = cfg->ffn;
        p.Fs = cfg->shared_ffn;
        p.E = cfg->n_experts;
        p.k = cfg->top_k;
        p.logits = logits;
        p.x = static_cast<const uint16_t*>(x);
        p.gate = static_cast<const uint8_t*>(w->gate);
        p.up = static_cast<const uint8_t*>(w->up);
        p.down = static_cast<const uint8_t*>(w->down);
        p.gate_s = static_cast<const uint8_t*>(w->gate_scales);
        p.up_s = static_cast<const uint8_t*>(w->up_scales);
        p.down_s = static_cast<const uint8_t*>(w->down_scales);
        p.sh_gate = static_cast<const uint16_t*>(w->sh_gate);
        p.sh_up = static_cast<const uint16_t*>(w->sh_up);
        p.sh_down = static_cast<const uint16_t*>(w->sh_down);
        p.h = reinterpret_cast<uint16_t*>(ws + L.h);
        p.sh_h = reinterpret_cast<uint16_t*>(ws + L.shh);
        p.y = static_cast<uint16_t*>(y);
        p.sel = reinterpret_cast<int32_t*>(ws + L.idx);
        p.selw = reinterpret_cast<float*>(ws + L.w);
        return hip_status(ds4::launch_layer_t1(p, s), "forward: batch-1 layer");
    }
    int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
    float* tw = reinterpret_cast<float*>(ws + L.w);
    int32_t* off = reinterpret_cast<int32_t*>(ws + L.off);
    int32_t* sp = reinterpret_cast<int32_t*>(ws + L.sp);
    int32_t* pp = reinterpret_cast<int32_t*>(ws + L.pp);
    int32_t* act = reinterpret_cast<int32_t*>(ws + L.act);
    void* eo = ws + L.eo;
    void* so = cfg->shared_ffn > 0 ? static_cast<void*>(ws + L.so) : nullptr;
    hipError_t e = ds4::launch_route(logits, T, cfg->n_experts, cfg->top_k, idx, tw, s);
    if (e != hipSuccess) return hip_status(e, "forward: route");
    if (T >= PERMUTE_BLOCKED_MIN_TOKENS)
        e = ds4::launch_permute_blocked(idx, T, cfg->n_experts, cfg->top_k, off, sp, pp, act,
                                        reinterpret_cast<int32_t*>(ws + L.perm), s);
    else
        e = ds4::launch_permute(idx, T, cfg->n_experts, cfg->top_k, off, sp, pp, act, s);
    if (e != hipSuccess) return hip_status(e, "forward: permute");
    TRY(run_ffn(cfg, w, T, x, off, sp, act, eo, so, workspace, s));
    return hip_status(ds4::launch_combine(cfg->act_dtype == DS4MOE_DT_BF16, T, cfg->hidden, cfg->top_k, eo, pp, tw,
                                          so, y, s),
                      "forward: combine");
}

size_t ds4moe_forward_noalloc_max_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

int ds4moe_forward_noalloc(const ds4moe_config* cfg, const ds4moe_weights* w, int32_t T, const void* x,
                           const float* logits, void* y, void* stream) {
    TRY(check_cfg(cfg));
    TRY(check_T(cfg, T));
    const size_t need = ws_layout(cfg, T).total;
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(DS4MOE_E_WORKSPACE, "forward_noalloc: this layer at T = %d needs %zu bytes of scratch, above the "
                    "library's fixed %zu", T, need, NOALLOC_SCRATCH_BYTES);
    int st = DS4MOE_OK;
    void* ws = scratch_for_current_device(&st);
    if (!ws) return st;
    return ds4moe_forward(cfg, w, T, x, logits, y, ws, NOALLOC_SCRATCH_BYTES, stream);
}

int ds4moe_quantize_mxfp8(const void* x_bf16, int64_t n, uint8_t* codes, uint8_t* scales, void* stream) {
    ds4::stage_call_begin();
    if (n < 0 || n % 32 || n > ((int64_t)1 << 40))
        return fail(DS4MOE_E_SHAPE, "n %lld must be a non-negative multiple of 32", (long long)n);
    REQ_PTR(x_bf16);
    REQ_PTR(codes);
    if (!scales) return fail(DS4MOE_E_ARG, "scales is NULL");
    return hip_status(ds4::launch_quantize_mx8(static_cast<const uint16_t*>(x_bf16), n, codes, scales,
                                               static_cast<hipStream_t>(stream)),
                      "quantize MXFP8");
}

int ds4moe_dequantize(int32_t wfmt, const void* data, const void* scales, int64_t n, float* out_f32,
                      uint16_t* out_bf16, void* stream) {
    ds4::stage_call_begin();
    if (wfmt != DS4MOE_WFMT_Q2K && wfmt != DS4MOE_WFMT_MXFP4 && wfmt != DS4MOE_WFMT_BF16 && wfmt != DS4MOE_WFMT_Q4K)
        return fail(DS4MOE_E_ARG, "wfmt %d", wfmt);
    const int64_t unit = (wfmt == DS4MOE_WFMT_Q2K || wfmt == DS4MOE_WFMT_Q4K) ? 256 : (wfmt == DS4MOE_WFMT_MXFP4 ? 32 : 16);
    if (n < 0 || n % unit || n > ((int64_t)1 << 40))
        return fail(DS4MOE_E_SHAPE, "n %lld must be a non-negative multiple of %lld", (long long)n, (long long)unit);
    REQ_PTR(data);
    if (wfmt == DS4MOE_WFMT_MXFP4 || wfmt == DS4MOE_WFMT_Q4K) {
        if (!scales) return fail(DS4MOE_E_ARG, "scales is NULL");
        if (wfmt == DS4MOE_WFMT_MXFP4 && !aligned16(scales)) return fail(DS4MOE_E_ALIGN, "scales not 16-byte aligned");
        if (wfmt == DS4MOE_WFMT_Q4K && (reinterpret_cast<uintptr_t>(scales) & 3u))
            return fail(DS4MOE_E_ALIGN, "Q4K parameters not 4-byte aligned");
    } else if (scales) {
        return fail(DS4MOE_E_ARG, "scales must be NULL unless wfmt is MXFP4 or Q4K");
    }
    if (!out_f32 && !out_bf16) return fail(DS4MOE_E_ARG, "both outputs are NULL");
    OPT_PTR(out_f32);
    OPT_PTR(out_bf16);
    return hip_status(ds4::launch_dequantize(wfmt, static_cast<const uint8_t*>(data),
                                             static_cast<const uint8_t*>(scales), n, out_f32, out_bf16,
                                             static_cast<hipStream_t>(stream)),
                      "dequantize");
}

}  // extern "C"
