"""The C ABI without a GPU: the library loads, exports every symbol that
include/ds4moe.h declares, and rejects bad arguments on the host before any
launch (so these calls never reach the device)."""
import ctypes
import os
import re

import pytest

ds4 = pytest.importorskip("bit_routed_moe_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4moe.h")
FAKE = 0x100000          # aligned, never dereferenced: every call below fails validation first
MIS = 0x100004           # 4-byte aligned only


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds4moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert _declared() == sorted(ds4.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(ds4.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    assert ds4.status_string(0) == "ok"
    for st in range(-6, 0):
        assert ds4.status_string(st) != "unknown status"
    assert "gfx950" in ds4.version()


def _cfg(**kw):
    base = dict(hidden=7168, ffn=2048, n_experts=256, top_k=8, shared_ffn=2048)
    base.update(kw)
    return ds4.make_config(**base)


def _status(fn, *args):
    st = fn(*args)
    msg = ds4.lib.ds4moe_last_error().decode()
    return st, msg


def test_route_validation():
    r = ds4.lib.ds4moe_route
    c = ctypes.byref
    assert _status(r, c(_cfg(top_k=0)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    assert _status(r, c(_cfg(top_k=65)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    assert _status(r, c(_cfg(n_experts=4, top_k=5)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    assert _status(r, c(_cfg(n_experts=1025)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    assert _status(r, c(_cfg()), 0, FAKE, FAKE, FAKE, 0)[0] == -2             # T = 0: empty input
    assert _status(r, c(_cfg()), -3, FAKE, FAKE, FAKE, 0)[0] == -2
    st, msg = _status(r, c(_cfg()), 1, None, FAKE, FAKE, 0)
    assert st == -1 and "logits" in msg
    assert _status(r, c(_cfg()), 1, MIS, FAKE, FAKE, 0)[0] == -3
    assert _status(r, None, 1, FAKE, FAKE, FAKE, 0)[0] == -1


def test_config_validation():
    r = ds4.lib.ds4moe_route
    c = ctypes.byref
    assert _status(r, c(_cfg(hidden=7000)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    assert _status(r, c(_cfg(ffn=100)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    assert _status(r, c(_cfg(shared_ffn=100)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    bad = _cfg()
    bad.wfmt = 9
    assert _status(r, c(bad), 1, FAKE, FAKE, FAKE, 0)[0] == -1
    bad = _cfg(wfmt="bf16")
    assert _status(r, c(bad), 1, FAKE, FAKE, FAKE, 0)[0] == -4
    bad = _cfg(act="f32", algo="grouped")
    assert _status(r, c(bad), 1, FAKE, FAKE, FAKE, 0)[0] == -4
    bad = _cfg()
    bad.algo = 7
    assert _status(r, c(bad), 1, FAKE, FAKE, FAKE, 0)[0] == -1
    bad = _cfg()
    bad.mma_dtype = 5
    assert _status(r, c(bad), 1, FAKE, FAKE, FAKE, 0)[0] == -1


def test_fp8_operand_config():
    """fp8 matrix-core operands: MXFP4 routed experts in the bf16 path on the
    grouped GEMM only; the batch-1 launches are bf16-operand kernels."""
    r = ds4.lib.ds4moe_route
    c = ctypes.byref
    ok = _cfg(wfmt="mxfp4", mma="fp8")
    assert _status(r, c(ok), 1, FAKE, FAKE, FAKE, 0)[0] != -4
    for kw in (dict(wfmt="q2k"), dict(wfmt="mxfp4", act="f32"), dict(wfmt="mxfp4", algo="gemv")):
        st, msg = _status(r, c(_cfg(mma="fp8", **kw)), 1, FAKE, FAKE, FAKE, 0)
        assert st == -4 and "fp8" in msg
    assert ds4.lib.ds4moe_forward_path(c(ok), 1) == 2
    assert ds4.lib.ds4moe_forward_path(c(_cfg(wfmt="mxfp4")), 1) == 1
    # E4M3 codes of x and E8M0 scales of x and h on top of the bf16 layout
    T = 4096
    extra = ds4.workspace_bytes(ok, T) - ds4.workspace_bytes(_cfg(wfmt="mxfp4"), T)
    assert extra >= T * 7168 + T * 7168 // 32 + T * 8 * 2048 // 32


def test_quantize_mxfp8_validation():
    q = ds4.lib.ds4moe_quantize_mxfp8
    assert _status(q, FAKE, 48, FAKE, FAKE, 0)[0] == -2
    assert _status(q, FAKE, -32, FAKE, FAKE, 0)[0] == -2
    assert _status(q, None, 32, FAKE, FAKE, 0)[0] == -1
    assert _status(q, FAKE, 32, None, FAKE, 0)[0] == -1
    assert _status(q, FAKE, 32, FAKE, None, 0)[0] == -1
    assert _status(q, MIS, 32, FAKE, FAKE, 0)[0] == -3


def test_forward_path_validation_and_general_path():
    """Invalid configurations are refused before any device query; more than
    one token, fp32 mode or a forced kernel choice take the general launches."""
    fp = ds4.lib.ds4moe_forward_path
    c = ctypes.byref
    assert fp(c(_cfg(hidden=7000)), 1) == -2
    assert fp(None, 1) == -1
    assert fp(c(_cfg()), 0) == -2
    assert fp(c(_cfg()), 2) == 0
    assert fp(c(_cfg()), 8) == 0            # AUTO: GEMV up to 8 tokens
    assert fp(c(_cfg()), 9) == 2            # grouped GEMM above
    assert fp(c(_cfg()), 4096) == 2
    assert fp(c(_cfg(act="f32")), 1) == 0
    assert fp(c(_cfg(act="f32")), 4096) == 0
    assert fp(c(_cfg(algo="gemv")), 1) == 0
    assert fp(c(_cfg(algo="grouped")), 1) == 2


def test_forward_validation():
    f = ds4.lib.ds4moe_forward
    c = ctypes.byref
    cfg = _cfg()
    w = ds4.Weights(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE)
    need = ds4.workspace_bytes(cfg, 4)
    assert need > 0
    assert _status(f, c(cfg), c(w), 4, FAKE, FAKE, FAKE, FAKE, need - 1, 0)[0] == -5
    assert _status(f, c(cfg), c(w), 4, FAKE, FAKE, FAKE, None, need, 0)[0] == -5
    assert _status(f, c(cfg), c(w), 4, FAKE, FAKE, FAKE, MIS, need, 0)[0] == -3
    w_noshared = ds4.Weights(FAKE, FAKE, FAKE, None, None, None, None, None, None)
    assert _status(f, c(cfg), c(w_noshared), 4, FAKE, FAKE, FAKE, FAKE, need, 0)[0] == -1
    w_scales = ds4.Weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert _status(f, c(cfg), c(w_scales), 4, FAKE, FAKE, FAKE, FAKE, need, 0)[0] == -1
    mx = _cfg(wfmt="mxfp4")
    assert _status(f, c(mx), c(w), 4, FAKE, FAKE, FAKE, FAKE, ds4.workspace_bytes(mx, 4), 0)[0] == -1
    w_mis = ds4.Weights(MIS, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE)
    assert _status(f, c(cfg), c(w_mis), 4, FAKE, FAKE, FAKE, FAKE, need, 0)[0] == -3
    assert _status(f, c(cfg), None, 4, FAKE, FAKE, FAKE, FAKE, need, 0)[0] == -1


def test_workspace_bytes():
    cfg = _cfg()
    a = ds4.workspace_bytes(cfg, 1)
    b = ds4.workspace_bytes(cfg, 4096)
    assert 0 < a < b
    # bf16 intermediates: h (T*k*F) + expert_out (T*k*H) dominate
    assert b >= 4096 * 8 * (2048 + 7168) * 2
    assert ds4.workspace_bytes(_cfg(top_k=0), 4) == 0
    assert ds4.workspace_bytes(cfg, 0) == 0


def test_dequantize_validation():
    d = ds4.lib.ds4moe_dequantize
    assert _status(d, 1, FAKE, None, 255, FAKE, None, 0)[0] == -2
    assert _status(d, 2, FAKE, None, 64, FAKE, None, 0)[0] == -1      # MXFP4 without scales
    assert _status(d, 1, FAKE, FAKE, 256, FAKE, None, 0)[0] == -1     # Q2K with scales
    assert _status(d, 1, FAKE, None, 256, None, None, 0)[0] == -1
    assert _status(d, 7, FAKE, None, 256, FAKE, None, 0)[0] == -1
    assert _status(d, 1, MIS, None, 256, FAKE, None, 0)[0] == -3


def test_expert_ffn_and_combine_validation():
    e = ds4.lib.ds4moe_expert_ffn
    cb = ds4.lib.ds4moe_combine
    c = ctypes.byref
    cfg = _cfg()
    w = ds4.Weights(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE)
    need = ds4.workspace_bytes(cfg, 2)
    assert _status(e, c(cfg), c(w), 2, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, 0)[0] == -1
    assert _status(e, c(cfg), c(w), 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 0)[0] == -5
    assert _status(cb, c(cfg), 2, FAKE, FAKE, FAKE, FAKE, None, 0)[0] == -1
    assert _status(cb, c(cfg), 2, FAKE, FAKE, FAKE, MIS, FAKE, 0)[0] == -3


def test_router_logits_validation():
    r = ds4.lib.ds4moe_router_logits
    c = ctypes.byref
    assert _status(r, c(_cfg(hidden=7000)), 1, FAKE, FAKE, FAKE, 0)[0] == -2
    assert _status(r, c(_cfg()), 0, FAKE, FAKE, FAKE, 0)[0] == -2
    st, msg = _status(r, c(_cfg()), 1, None, FAKE, FAKE, 0)
    assert st == -1 and "x" in msg
    st, msg = _status(r, c(_cfg()), 1, FAKE, None, FAKE, 0)
    assert st == -1 and "router_w" in msg
    assert _status(r, c(_cfg()), 1, FAKE, FAKE, None, 0)[0] == -1
    assert _status(r, c(_cfg()), 1, FAKE, MIS, FAKE, 0)[0] == -3
    assert _status(r, None, 1, FAKE, FAKE, FAKE, 0)[0] == -1


def test_workspace_regions():
    """Forward's stage results sit at 256-byte offsets inside the workspace,
    do not overlap, and have the sizes their layouts give."""
    for cfg, T in ((_cfg(), 4096), (_cfg(), 1), (ds4.make_config(256, 128, 1024, 8, 0, act="f32"), 300)):
        total = ds4.workspace_bytes(cfg, T)
        k, E, H = cfg.top_k, cfg.n_experts, cfg.hidden
        eb = 4 if cfg.act_dtype == 0 else 2
        want = {"topk_idx": T * k * 4, "topk_w": T * k * 4, "offsets": (E + 1) * 4, "sorted_pair": T * k * 4,
                "pair_pos": T * k * 4, "active": (E + 1) * 4, "expert_out": T * k * H * eb,
                "shared_out": T * H * eb}
        spans = []
        for name, n in want.items():
            off, got = ds4.workspace_region(cfg, T, name)
            assert got == n, name
            assert off % 256 == 0 and off + got <= total, name
            spans.append((off, off + got))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    with pytest.raises(ds4.Ds4MoeError):
        ds4.workspace_region(_cfg(), 4, 8)
    with pytest.raises(ds4.Ds4MoeError):
        ds4.workspace_region(_cfg(top_k=0), 4, 0)


def test_width_limits():
    """hidden, ffn and shared_ffn above 32768 are refused on the host: at such
    widths some kernel's activation staging would not fit a workgroup's LDS."""
    c = ctypes.byref
    for kw in (dict(hidden=32768 + 256), dict(ffn=32768 + 128), dict(shared_ffn=32768 + 128)):
        st, msg = _status(ds4.lib.ds4moe_forward_path, c(_cfg(**kw)), 1)
        assert st == -2, (kw, st, msg)
    assert ds4.lib.ds4moe_forward_path(c(_cfg(hidden=32768, ffn=32768, shared_ffn=32768)), 1) >= 0
