"""Seeded synthetic inputs for the one-GPU MoE layer (router -> drop -> permute ->
grouped SwiGLU expert FFN -> gate-weighted un-permute, forward and backward).

This module only draws random tensors with the shapes, distributions and seeds of
the five layer shapes below. It holds none of the layer's arithmetic, so both the
HIP path and the CPU oracle can take their inputs from it without sharing code.

Recipe (one torch.Generator per tensor, so each tensor is reproducible on its own):
  generator = torch.Generator(device).manual_seed(seed * 1000 + slot)
  value     = torch.randn(shape, generator, float32) * std
  bf16 cfgs : value.to(bfloat16)  (round-to-nearest-even), the rounded tensor is the input
Slots, in order: x, w_router, w_gate, w_up, w_down, dy, w_sg (shared-gate vector),
ws_gate, ws_up, ws_down (shared expert).  Weights of the routed experts are drawn one
expert at a time (slot * 1000 + 100 + e) to bound memory.  The Zipf router bias of the
fine-grained shape is b_e = 1.5 * ln(1 / (e + 1)), computed in float64 and stored as fp32.

Weight layouts (y = x . W): w_router [d, E]; w_gate, w_up [E, d, f]; w_down [E, f, d];
w_sg [d]; ws_gate, ws_up [1, d, fs]; ws_down [1, fs, d].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["LayerShape", "SHAPES", "shape_by_name", "make_inputs", "make_router_inputs", "ShardShape", "SHARDS",
           "shard_by_name", "make_source_tokens", "make_shard_weights", "make_shard_grad"]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    T: int            # tokens on this GPU
    d: int            # hidden size
    E: int            # routed experts
    K: int            # experts per token (top-K)
    f: int            # SwiGLU ffn size per routed expert
    seed: int
    dtype: str        # "f32" or "bf16"
    cf: Optional[float]   # capacity factor; None = dropless
    sub_seq: int      # sub-sequence length S used by the drop rule (T % S == 0)
    w_std: Optional[float]  # std of expert weights; None = 1/sqrt(fan_in)
    wr_std: float     # std of the router weight
    fs: int = 0       # shared-expert ffn size (0 = no shared expert)
    zipf_bias: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


SHAPES = [
    # Tiny top-2 layer, fp32, dropless.
    LayerShape("tiny", T=256, d=64, E=4, K=2, f=128, seed=0, dtype="f32", cf=None,
               sub_seq=256, w_std=None, wr_std=0.02),
    # Mixtral-8x22B-shaped layer, one 4096-token sub-sequence, capacity factor 1.0.
    LayerShape("mixtral_8x22b", T=4096, d=6144, E=8, K=2, f=16384, seed=1, dtype="bf16",
               cf=1.0, sub_seq=4096, w_std=0.02, wr_std=0.02),
    # Qwen2-57B-A14B-shaped fine-grained layer with a sigmoid-gated shared expert, dropless.
    LayerShape("qwen2_57b_a14b", T=4096, d=3584, E=64, K=8, f=2560, seed=2, dtype="bf16",
               cf=None, sub_seq=4096, w_std=0.02, wr_std=0.02, fs=20480),
    # Mixtral-8x22B-G8T8 shape, capacity factor 1.0, Zipf-skewed router bias.
    LayerShape("mixtral_g8t8", T=4096, d=6144, E=64, K=8, f=2048, seed=3, dtype="bf16",
               cf=1.0, sub_seq=4096, w_std=0.02, wr_std=0.02, zipf_bias=True),
    # Llama3-8x70B-shaped layer, one GPU's 8192-token share of a 128K sequence, dropless.
    LayerShape("llama3_8x70b", T=8192, d=8192, E=8, K=2, f=28672, seed=4, dtype="bf16",
               cf=None, sub_seq=8192, w_std=0.02, wr_std=0.02),
    # Mixtral-8x22B dimensions over 16384 tokens dropped per 4096-token sub-sequence
    # (capacity 1024 per sub-sequence and expert) ...
    LayerShape("mixtral_t16k_s4k", T=16384, d=6144, E=8, K=2, f=16384, seed=5, dtype="bf16",
               cf=1.0, sub_seq=4096, w_std=0.02, wr_std=0.02),
    # ... and the same tokens dropped over the full sequence (capacity 4096 per expert).
    LayerShape("mixtral_t16k_full", T=16384, d=6144, E=8, K=2, f=16384, seed=5, dtype="bf16",
               cf=1.0, sub_seq=16384, w_std=0.02, wr_std=0.02),
]


def shape_by_name(name: str) -> LayerShape:
    for s in SHAPES:
        if s.name == name:
            return s
    raise KeyError(name)


_SLOT = {"x": 0, "w_router": 1, "w_gate": 2, "w_up": 3, "w_down": 4, "dy": 5,
         "w_sg": 6, "ws_gate": 7, "ws_up": 8, "ws_down": 9}


def _randn(shape, seed: int, slot: int, std: float, dtype, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + slot)
    t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _expert_stack(E, rows, cols, seed, slot, std, dtype, device) -> torch.Tensor:
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    for e in range(E):
        out[e] = _randn((rows, cols), seed, slot * 1000 + 100 + e, std, dtype, device)
    return out


def make_inputs(shape: LayerShape, device="cpu", T: Optional[int] = None,
                with_shared: Optional[bool] = None) -> dict:
    """Draw every input tensor of one layer shape on `device`.

    `T` overrides the token count (same seeds, a shorter x/dy) for reduced-size cases.
    Returns a dict of tensors (bias is None unless the shape has the Zipf bias).
    """
    s = shape
    T = s.T if T is None else T
    dt = s.torch_dtype
    g_std = s.w_std if s.w_std is not None else 1.0 / math.sqrt(s.d)
    d_std = s.w_std if s.w_std is not None else 1.0 / math.sqrt(s.f)
    out = {
        "x": _randn((T, s.d), s.seed, _SLOT["x"], 1.0, dt, device),
        "w_router": _randn((s.d, s.E), s.seed, _SLOT["w_router"], s.wr_std, dt, device),
        "w_gate": _expert_stack(s.E, s.d, s.f, s.seed, _SLOT["w_gate"], g_std, dt, device),
        "w_up": _expert_stack(s.E, s.d, s.f, s.seed, _SLOT["w_up"], g_std, dt, device),
        "w_down": _expert_stack(s.E, s.f, s.d, s.seed, _SLOT["w_down"], d_std, dt, device),
        "dy": _randn((T, s.d), s.seed, _SLOT["dy"], 1.0, dt, device),
        "bias": None,
    }
    if s.zipf_bias:
        b = torch.tensor([1.5 * math.log(1.0 / (e + 1)) for e in range(s.E)],
                         dtype=torch.float64).to(torch.float32)
        out["bias"] = b.to(device)
    shared = (s.fs > 0) if with_shared is None else with_shared
    if shared and s.fs > 0:
        out["w_sg"] = _randn((s.d,), s.seed, _SLOT["w_sg"], s.w_std, dt, device)
        out["ws_gate"] = _expert_stack(1, s.d, s.fs, s.seed, _SLOT["ws_gate"], s.w_std, dt, device)
        out["ws_up"] = _expert_stack(1, s.d, s.fs, s.seed, _SLOT["ws_up"], s.w_std, dt, device)
        out["ws_down"] = _expert_stack(1, s.fs, s.d, s.seed, _SLOT["ws_down"], s.w_std, dt, device)
    return out


def make_router_inputs(shape: LayerShape, device="cpu") -> dict:
    """Only the router's inputs of a layer shape (x, w_router, bias), drawn exactly as
    make_inputs draws them; the expert weights are not drawn."""
    s = shape
    dt = s.torch_dtype
    out = {"x": _randn((s.T, s.d), s.seed, _SLOT["x"], 1.0, dt, device),
           "w_router": _randn((s.d, s.E), s.seed, _SLOT["w_router"], s.wr_std, dt, device),
           "bias": None}
    if s.zipf_bias:
        b = torch.tensor([1.5 * math.log(1.0 / (e + 1)) for e in range(s.E)],
                         dtype=torch.float64).to(torch.float32)
        out["bias"] = b.to(device)
    return out


# --------------------------------------------------------------------------------------
# One GPU's expert-side share of a layer spread over G GPUs
# --------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ShardShape:
    """The experts one GPU holds when the layer `source` runs on G GPUs.

    Each of the G GPUs routes its own T tokens (one sub-sequence per GPU, so the drop is
    per source); the rows routed to experts [e0, e1) reach this GPU.  With etp > 1 the
    GPU holds the ffn slice [etp_rank * f / etp, (etp_rank + 1) * f / etp) of each of
    those experts and its o and dxp are partial sums over the slice.

    Recipe: x of all G sources is one [G * T, d] tensor drawn like a layer's x (same
    seed and slot, G * T rows); the router weight is the source layer's; the local
    weights are the source layer's expert weights (same per-expert seeds), sliced; the
    output gradient of the received rows is drawn with the dy slot and seed * 1000 + 500.
    """
    name: str
    source: str
    G: int
    e0: int
    e1: int
    etp: int = 1
    etp_rank: int = 0

    @property
    def layer(self) -> LayerShape:
        return shape_by_name(self.source)

    @property
    def E_local(self) -> int:
        return self.e1 - self.e0

    @property
    def f_local(self) -> int:
        return self.layer.f // self.etp

    @property
    def cols(self) -> slice:
        return slice(self.etp_rank * self.f_local, (self.etp_rank + 1) * self.f_local)


SHARDS = [
    # Mixtral-8x22B layer over 8 GPUs (8 x 4096 tokens), capacity factor 1.0:
    # EP 8: one expert per GPU, its rows from all 8 GPUs;
    ShardShape("mixtral_ep8", "mixtral_8x22b", G=8, e0=0, e1=1),
    # EP 4 x ETP 2: two experts per GPU, half of their ffn;
    ShardShape("mixtral_ep4_etp2", "mixtral_8x22b", G=8, e0=0, e1=2, etp=2),
    # ETP 8: every expert, an eighth of its ffn.
    ShardShape("mixtral_etp8", "mixtral_8x22b", G=8, e0=0, e1=8, etp=8),
]


def shard_by_name(name: str) -> ShardShape:
    for s in SHARDS:
        if s.name == name:
            return s
    raise KeyError(name)


def make_source_tokens(shape: LayerShape, G: int, device="cpu") -> dict:
    """x of G source GPUs ([G * T, d], drawn as one tensor) and the router's inputs."""
    s = shape
    dt = s.torch_dtype
    out = {
        "x": _randn((G * s.T, s.d), s.seed, _SLOT["x"], 1.0, dt, device),
        "w_router": _randn((s.d, s.E), s.seed, _SLOT["w_router"], s.wr_std, dt, device),
        "bias": None,
    }
    if s.zipf_bias:
        b = torch.tensor([1.5 * math.log(1.0 / (e + 1)) for e in range(s.E)],
                         dtype=torch.float64).to(torch.float32)
        out["bias"] = b.to(device)
    return out


def make_shard_weights(shard: ShardShape, device="cpu", layer: Optional[LayerShape] = None) -> dict:
    """The local experts' weights, ffn-sliced: w_gate, w_up [E_local, d, f_local] and
    w_down [E_local, f_local, d], each expert drawn in full with its own seed."""
    s = layer or shard.layer
    dt = s.torch_dtype
    g_std = s.w_std if s.w_std is not None else 1.0 / math.sqrt(s.d)
    d_std = s.w_std if s.w_std is not None else 1.0 / math.sqrt(s.f)
    fl, c = s.f // shard.etp, slice(shard.etp_rank * (s.f // shard.etp),
                                    (shard.etp_rank + 1) * (s.f // shard.etp))
    El = shard.e1 - shard.e0
    out = {"w_gate": torch.empty((El, s.d, fl), dtype=dt, device=device),
           "w_up": torch.empty((El, s.d, fl), dtype=dt, device=device),
           "w_down": torch.empty((El, fl, s.d), dtype=dt, device=device)}
    for i, e in enumerate(range(shard.e0, shard.e1)):
        for key, slot, shp, std in (("w_gate", "w_gate", (s.d, s.f), g_std),
                                    ("w_up", "w_up", (s.d, s.f), g_std),
                                    ("w_down", "w_down", (s.f, s.d), d_std)):
            w = _randn(shp, s.seed, _SLOT[slot] * 1000 + 100 + e, std, dt, device)
            out[key][i] = w[:, c] if key != "w_down" else w[c, :]
            del w
    return out


def make_shard_grad(shard: ShardShape, rows: int, device="cpu",
                    layer: Optional[LayerShape] = None) -> torch.Tensor:
    """Gradient of the received rows' expert outputs, [rows, d]."""
    s = layer or shard.layer
    return _randn((rows, s.d), s.seed * 1000 + 500, _SLOT["dy"], 1.0, s.torch_dtype, device)
