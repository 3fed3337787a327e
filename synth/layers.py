"""Seeded synthetic MoE layers, activations and router logits.

Recipe (every draw is seeded; see ``derive_seed``):
  * routed gate/up/down weights ~ N(0, 0.02), encoded to Q2K-style blocks,
    Q4K-style blocks or MXFP4 by ``synth.quant``; gate/up are [E][F][H], down
    is [E][H][F]
    (rows x contraction dim, row-major);
  * shared-expert gate/up [Fs][H] and down [H][Fs] ~ N(0, 0.02) rounded to bf16
    (the pages keep the shared expert at original precision: hysenlabs
    "DwarfStar実地分析", section "GGUFの対応範囲は意図的に狭い");
  * activations x ~ N(0, 1) (fp32, or rounded to bf16);
  * router logits ~ N(0, 1) fp32, optionally plus a per-expert Zipf(s) bias
    b_e = ln p_rank(e), p_r proportional to r**-s, ranks given to experts by a
    seeded permutation, logits = fp32(z + b).

Small layers are drawn with numpy on the host; full-size layers are drawn with
torch generators on the device they are made for (bytes are reproducible per
device type, and the oracle always reads the bytes actually made).
"""
from dataclasses import dataclass, field
import hashlib
import numpy as np
import torch

from .quant import q2k_encode, mxfp4_encode, q4k_encode

BASE_SEED = 20261202
_MATS = ("gate", "up", "down", "sh_gate", "sh_up", "sh_down", "x", "logits", "zipf")


def derive_seed(base: int, copy: int, what: str, index: int = 0) -> int:
    """Deterministic 63-bit seed for (base seed, layer copy, tensor name, index)."""
    h = hashlib.sha256(f"{base}/{copy}/{what}/{index}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


@dataclass(frozen=True)
class LayerSpec:
    hidden: int
    ffn: int
    n_experts: int
    top_k: int
    shared_ffn: int = 0
    wfmt: str = "q2k"          # "q2k" | "mxfp4" | "q4k"

    def routed_shape(self, name: str):
        return (self.ffn, self.hidden) if name in ("gate", "up") else (self.hidden, self.ffn)

    def shared_shape(self, name: str):
        return (self.shared_ffn, self.hidden) if name in ("sh_gate", "sh_up") else (self.hidden, self.shared_ffn)


@dataclass
class Layer:
    """Encoded layer.  Tensors live on ``device``.

    Q2K:   gate/up/down uint8 [E][rows*K/256*84]; *_scales None.
    MXFP4: gate/up/down uint8 [E][rows][K/2]; gate_scales/... uint8 [E][rows][K/32].
    Q4K:   gate/up/down uint8 [E][rows][K/2]; gate_scales/... uint8 [E][rows][K/256][20].
    Shared: sh_gate/sh_up/sh_down bfloat16 (None when shared_ffn == 0).
    """
    spec: LayerSpec
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    gate_scales: torch.Tensor = None
    up_scales: torch.Tensor = None
    down_scales: torch.Tensor = None
    sh_gate: torch.Tensor = None
    sh_up: torch.Tensor = None
    sh_down: torch.Tensor = None
    _host_cache: dict = field(default_factory=dict, repr=False)

    @property
    def device(self):
        return self.gate.device

    # ---- host views used by the oracle (data access only) -----------------
    def routed(self, name: str, e: int):
        """Host copy of expert ``e``'s bytes for matrix ``name``:
        (data uint8 ndarray, scales uint8 ndarray or None)."""
        key = (name, e)
        hit = self._host_cache.get(key)
        if hit is not None:
            return hit
        data = getattr(self, name)[e].cpu().numpy()
        sc = getattr(self, name + "_scales")
        sc = None if sc is None else sc[e].cpu().numpy()
        if len(self._host_cache) > 64:
            self._host_cache.clear()
        self._host_cache[key] = (data, sc)
        return data, sc

    def shared(self, name: str):
        """Host copy of a shared-expert matrix as bf16 bit patterns (uint16), or None."""
        t = getattr(self, name)
        if t is None:
            return None
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    def clone(self) -> "Layer":
        kw = {}
        for f in ("gate", "up", "down", "gate_scales", "up_scales", "down_scales",
                  "sh_gate", "sh_up", "sh_down"):
            t = getattr(self, f)
            kw[f] = None if t is None else t.clone()
        return Layer(spec=self.spec, **kw)

    def weight_bytes(self) -> dict:
        out = {}
        for f in ("gate", "up", "down", "gate_scales", "up_scales", "down_scales",
                  "sh_gate", "sh_up", "sh_down"):
            t = getattr(self, f)
            out[f] = 0 if t is None else t.numel() * t.element_size()
        return out


def _normal(shape, std, seed, device, host_rng: bool):
    if host_rng:
        rng = np.random.default_rng(seed)
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).to(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def make_layer(spec: LayerSpec, seed: int = BASE_SEED, copy: int = 0, device="cpu",
               host_rng=None, std: float = 0.02) -> Layer:
    """Draw and encode one layer.  ``host_rng`` (default: True for CPU) draws
    with numpy so CPU-made layers are identical on every machine."""
    device = torch.device(device)
    if host_rng is None:
        host_rng = device.type == "cpu"
    E = spec.n_experts
    kw = {}
    for name in ("gate", "up", "down"):
        rows, K = spec.routed_shape(name)
        datas, scales = [], []
        for e in range(E):
            w = _normal((rows, K), std, derive_seed(seed, copy, name, e), device, host_rng)
            if spec.wfmt == "q2k":
                datas.append(q2k_encode(w).reshape(-1))
            elif spec.wfmt == "mxfp4":
                c, s = mxfp4_encode(w)
                datas.append(c)
                scales.append(s)
            elif spec.wfmt == "q4k":
                c, s = q4k_encode(w)
                datas.append(c)
                scales.append(s)
            else:
                raise ValueError(spec.wfmt)
            del w
        kw[name] = torch.stack(datas)
        if scales:
            kw[name + "_scales"] = torch.stack(scales)
    if spec.shared_ffn:
        for name in ("sh_gate", "sh_up", "sh_down"):
            w = _normal(spec.shared_shape(name), std, derive_seed(seed, copy, name), device, host_rng)
            kw[name] = w.to(torch.bfloat16)
    return Layer(spec=spec, **kw)


def make_x(T: int, H: int, seed: int = BASE_SEED, copy: int = 0, dtype: str = "bf16") -> torch.Tensor:
    """Activations x ~ N(0,1) on the host, fp32 or rounded to bf16 (RNE)."""
    rng = np.random.default_rng(derive_seed(seed, copy, "x"))
    x = torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32))
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def make_router_w(E: int, H: int, seed: int = BASE_SEED, copy: int = 0) -> torch.Tensor:
    """Router matrix [E][H] ~ N(0, 1/H) rounded to bf16 (RNE) on the host, so
    that N(0,1) activations give logits of about unit variance."""
    rng = np.random.default_rng(derive_seed(seed, copy, "router_w"))
    w = rng.standard_normal((E, H), dtype=np.float32) * np.float32(H ** -0.5)
    return torch.from_numpy(w).to(torch.bfloat16)


def zipf_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Per-expert log-popularity b_e = ln p_rank(e), p_r ~ r**-s, r = 1..E."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    perm = np.random.default_rng(seed).permutation(E)   # perm[e] = rank-1 of expert e
    return np.log(p[perm])


def make_logits(T: int, E: int, seed: int = BASE_SEED, copy: int = 0, zipf_s: float = None,
                index: int = 0) -> torch.Tensor:
    """Router logits fp32 [T][E] ~ N(0,1) (+ Zipf bias) on the host."""
    rng = np.random.default_rng(derive_seed(seed, copy, "logits", index))
    z = rng.standard_normal((T, E))
    if zipf_s is not None:
        z = z + zipf_bias(E, zipf_s, derive_seed(seed, copy, "zipf"))[None, :]
    return torch.from_numpy(z.astype(np.float32))


# Workloads: the shapes and value mixes the library is measured and checked on.
WORKLOADS = {
    "tiny": dict(spec=LayerSpec(256, 128, 8, 2, 0, "q2k"), T=16, zipf=None,
                 desc="hidden 256, expert ffn 128, 8 experts top-2, no shared, 16 tokens"),
    "decode": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "q2k"), T=1, zipf=None,
                   desc="batch-1 decode, 7168/2048, 256 experts top-8 + bf16 shared expert"),
    "batched_decode": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "q2k"), T=32, zipf=1.1,
                           desc="32-token decode, Zipf(1.1) expert popularity"),
    "prefill": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "q2k"), T=4096, zipf=None,
                    desc="4096-token prefill chunk, uniform routing"),
    "mxfp4_decode": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "mxfp4"), T=1, zipf=None,
                         desc="batch-1 decode, MXFP4 routed experts"),
    "mxfp4_prefill": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "mxfp4"), T=4096, zipf=None,
                          desc="4096-token prefill, MXFP4 routed experts"),
    "q4k_decode": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "q4k"), T=1, zipf=None,
                       desc="batch-1 decode, Q4K (4-bit) routed experts"),
    "q4k_prefill": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "q4k"), T=4096, zipf=None,
                        desc="4096-token prefill, Q4K (4-bit) routed experts"),
    # small batches through the GEMV / grouped crossover
    "verify6": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "q2k"), T=6, zipf=None,
                    desc="6 tokens (1 + 5 speculative drafts) of one sequence, uniform routing"),
    "sessions16": dict(spec=LayerSpec(7168, 2048, 256, 8, 2048, "q2k"), T=16, zipf=1.1,
                       desc="16 concurrent sessions, Zipf(1.1) expert popularity"),
}


def workload(name: str) -> dict:
    return WORKLOADS[name]
