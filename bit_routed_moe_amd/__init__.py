"""ds4moe: one routed-MoE layer over low-bit experts on an AMD Instinct MI355X.

A thin ctypes binding over ``libds4moe.so`` (built from ``csrc/`` by
``bit_routed_moe_amd.build``).  Every function takes caller-allocated torch
tensors, passes their device pointers and the current HIP stream to the C ABI
of the same name (see ``include/ds4moe.h``), and raises ``Ds4MoeError`` on a
non-OK status.  Nothing here computes: every step runs in the HIP kernels.
There is no CPU fallback; importing the package fails if the library has not
been built.
"""
import ctypes
import os

__all__ = [
    "Config", "Weights", "Ds4MoeError", "WFMT", "DTYPE", "ALGO", "LIB_PATH", "lib",
    "make_config", "make_weights", "router_logits", "route", "permute", "expert_ffn", "combine", "forward",
    "forward_noalloc", "forward_noalloc_max_bytes",
    "workspace_bytes", "workspace_region", "WS_REGION", "dequantize", "quantize_mxfp8", "status_string", "version",
    "EXPORTS", "STAGE", "set_stage_events",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libds4moe.so")

WFMT = {"q2k": 1, "mxfp4": 2, "bf16": 3, "q4k": 4}
DTYPE = {"f32": 0, "bf16": 1, "fp8": 2}
ALGO = {"auto": 0, "gemv": 1, "grouped": 2}

# Every entry point declared in include/ds4moe.h.
EXPORTS = (
    "ds4moe_router_logits", "ds4moe_route", "ds4moe_permute", "ds4moe_expert_ffn", "ds4moe_combine", "ds4moe_forward",
    "ds4moe_workspace_bytes", "ds4moe_dequantize", "ds4moe_status_string", "ds4moe_last_error",
    "ds4moe_version", "ds4moe_set_stage_events", "ds4moe_forward_path", "ds4moe_quantize_mxfp8",
    "ds4moe_workspace_region", "ds4moe_forward_noalloc", "ds4moe_forward_noalloc_max_bytes",
)

WS_REGION = {"topk_idx": 0, "topk_w": 1, "offsets": 2, "sorted_pair": 3, "pair_pos": 4, "active": 5,
             "expert_out": 6, "shared_out": 7}

STAGE = {"route": 0, "permute": 1, "ffn_up": 2, "ffn_down": 3, "combine": 4, "router_proj": 5}


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "ffn", "n_experts", "top_k", "shared_ffn", "wfmt", "act_dtype", "mma_dtype", "algo")]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "gate", "up", "down", "gate_scales", "up_scales", "down_scales", "sh_gate", "sh_up", "sh_down")]


class Ds4MoeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"ds4moe status {status}: {message}")
        self.status = status


def _load():
    # torch's HIP runtime must be the process's runtime before the library is
    # mapped: the library's libamdhip64.so.7 dependency then resolves to
    # torch's copy, and torch's pointers and streams are valid in its launches.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_routed_moe_amd.build` "
                          "(hipcc, gfx950); there is no fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp, wp = ctypes.POINTER(Config), ctypes.POINTER(Weights)
    sigs = {
        "ds4moe_router_logits": (i32, [cfgp, i32, vp, vp, vp, vp]),
        "ds4moe_route": (i32, [cfgp, i32, vp, vp, vp, vp]),
        "ds4moe_permute": (i32, [cfgp, i32, vp, vp, vp, vp, vp, vp]),
        "ds4moe_expert_ffn": (i32, [cfgp, wp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "ds4moe_combine": (i32, [cfgp, i32, vp, vp, vp, vp, vp, vp]),
        "ds4moe_forward": (i32, [cfgp, wp, i32, vp, vp, vp, vp, sz, vp]),
        "ds4moe_workspace_bytes": (sz, [cfgp, i32]),
        "ds4moe_dequantize": (i32, [i32, vp, vp, i64, vp, vp, vp]),
        "ds4moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "ds4moe_last_error": (ctypes.c_char_p, []),
        "ds4moe_version": (ctypes.c_char_p, []),
        "ds4moe_set_stage_events": (i32, [ctypes.c_int, vp, vp]),
        "ds4moe_forward_path": (i32, [cfgp, i32]),
        "ds4moe_quantize_mxfp8": (i32, [vp, i64, vp, vp, vp]),
        "ds4moe_workspace_region": (i32, [cfgp, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "ds4moe_forward_noalloc": (i32, [cfgp, wp, i32, vp, vp, vp, vp]),
        "ds4moe_forward_noalloc_max_bytes": (sz, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def status_string(st: int) -> str:
    return lib.ds4moe_status_string(st).decode()


def version() -> str:
    return lib.ds4moe_version().decode()


def _check(st: int):
    if st != 0:
        raise Ds4MoeError(st, f"{status_string(st)}: {lib.ds4moe_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_config(hidden, ffn, n_experts, top_k, shared_ffn=0, wfmt="q2k", act="bf16", mma="bf16",
                algo="auto") -> Config:
    return Config(hidden, ffn, n_experts, top_k, shared_ffn, WFMT[wfmt], DTYPE[act], DTYPE[mma], ALGO[algo])


def make_weights(gate, up, down, gate_scales=None, up_scales=None, down_scales=None,
                 sh_gate=None, sh_up=None, sh_down=None) -> Weights:
    """Device tensors -> the pointer struct.  The caller keeps the tensors alive."""
    ptr = lambda t: None if t is None else t.data_ptr()
    return Weights(ptr(gate), ptr(up), ptr(down), ptr(gate_scales), ptr(up_scales), ptr(down_scales),
                   ptr(sh_gate), ptr(sh_up), ptr(sh_down))


def workspace_bytes(cfg: Config, T_max: int) -> int:
    return int(lib.ds4moe_workspace_bytes(ctypes.byref(cfg), T_max))


def workspace_region(cfg: Config, T: int, region) -> tuple:
    """(byte offset, byte count) of a stage result inside forward's workspace
    ("topk_idx", "topk_w", "offsets", "sorted_pair", "pair_pos", "active",
    "expert_out", "shared_out")."""
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    r = WS_REGION[region] if isinstance(region, str) else region
    _check(lib.ds4moe_workspace_region(ctypes.byref(cfg), T, r, ctypes.byref(off), ctypes.byref(n)))
    return int(off.value), int(n.value)


def router_logits(cfg, T, x, router_w, logits, stream=None):
    _check(lib.ds4moe_router_logits(ctypes.byref(cfg), T, _p(x), _p(router_w), _p(logits), _s(stream)))


def route(cfg, T, logits, topk_idx, topk_w, stream=None):
    _check(lib.ds4moe_route(ctypes.byref(cfg), T, _p(logits), _p(topk_idx), _p(topk_w), _s(stream)))


def permute(cfg, T, topk_idx, expert_offsets, sorted_pair, pair_pos, active, stream=None):
    _check(lib.ds4moe_permute(ctypes.byref(cfg), T, _p(topk_idx), _p(expert_offsets), _p(sorted_pair),
                              _p(pair_pos), _p(active), _s(stream)))


def expert_ffn(cfg, weights, T, x, expert_offsets, sorted_pair, active, expert_out, shared_out,
               workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ds4moe_expert_ffn(ctypes.byref(cfg), ctypes.byref(weights), T, _p(x), _p(expert_offsets),
                                 _p(sorted_pair), _p(active), _p(expert_out), _p(shared_out),
                                 _p(workspace), nbytes, _s(stream)))


def combine(cfg, T, expert_out, pair_pos, topk_w, shared_out, y, stream=None):
    _check(lib.ds4moe_combine(ctypes.byref(cfg), T, _p(expert_out), _p(pair_pos), _p(topk_w),
                              _p(shared_out), _p(y), _s(stream)))


def forward(cfg, weights, T, x, logits, y, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ds4moe_forward(ctypes.byref(cfg), ctypes.byref(weights), T, _p(x), _p(logits), _p(y),
                              _p(workspace), nbytes, _s(stream)))


def forward_noalloc(cfg, weights, T, x, logits, y, stream=None):
    """ds4moe_forward with its workspace in the library's fixed per-device
    array (no device allocation; overlapping calls on one device race)."""
    _check(lib.ds4moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), T, _p(x), _p(logits), _p(y),
                                      _s(stream)))


def forward_noalloc_max_bytes() -> int:
    return int(lib.ds4moe_forward_noalloc_max_bytes())


def forward_path(cfg, T):
    """1: batch 1 in two launches; else route/permute/FFN/combine launches
    with the expert FFNs on the GEMV kernels (0) or the grouped GEMM (2)."""
    st = lib.ds4moe_forward_path(ctypes.byref(cfg), T)
    if st < 0:
        _check(st)
    return st


def dequantize(wfmt, data, scales, n, out_f32=None, out_bf16=None, stream=None):
    _check(lib.ds4moe_dequantize(WFMT[wfmt] if isinstance(wfmt, str) else wfmt, _p(data), _p(scales), n,
                                 _p(out_f32), _p(out_bf16), _s(stream)))


def quantize_mxfp8(x, n, codes, scales, stream=None):
    """MXFP8-E4M3 codes [n] and E8M0 scales [n/32] of n bf16 values."""
    _check(lib.ds4moe_quantize_mxfp8(_p(x), n, _p(codes), _p(scales), _s(stream)))


def set_stage_events(stage, start=None, stop=None):
    """Record torch.cuda.Event pair (created with enable_timing=True and
    already recorded once, so that it has a HIP event handle) around every
    launch of `stage` ("route", "permute", "ffn_up", "ffn_down", "combine")
    on this thread; "router_proj" times ds4moe_router_logits; no events clears."""
    h = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)
    _check(lib.ds4moe_set_stage_events(STAGE[stage] if isinstance(stage, str) else stage, h(start), h(stop)))
