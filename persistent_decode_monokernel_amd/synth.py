"""Seeded synthetic inputs: model shapes, weights, prompts, KV caches, GEMV probes.

This module only draws random numbers and lays them out.  It holds none of the
decoder's arithmetic, so both the GPU path and the CPU oracle can be fed from
it without sharing any computation.

Recipe (all seeds fixed per workload):
  * weights ~ N(0, 0.02^2), drawn in float32 by ``torch.randn`` on the chosen
    device from ``torch.Generator(device).manual_seed(seed)``, scaled by 0.02,
    then rounded (round-to-nearest-even) to the storage dtype; tensors are drawn
    in one fixed order: tok_emb, then per layer attn_norm, wq, wk, wv, wo,
    ffn_norm, w_gate, w_up, w_down, then final_norm, lm_head;
  * RMSNorm gains are 1.0 unless ``gain_jitter`` > 0 (then 1 + jitter*N(0,1));
  * prompts: ids uniform in [0, vocab) from a CPU generator;
  * KV caches (for decode-only workloads): N(0, 1) in the storage dtype, which
    matches the scale of k = Wk.xn with |xn|_rms = 1 and std(W) = 0.02,
    d = 2048..4096.
The same seed on a different device gives a different (but fixed) stream.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import torch

F16 = 1
BF16 = 2


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    dtype: int = F16
    rms_eps: float = 1e-5
    rope_base: float = 10000.0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float16 if self.dtype == F16 else torch.bfloat16


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named decode workload: shape, prompt length, decode length, seeds."""
    name: str
    shape: ModelShape
    n_prompt: int
    n_decode: int
    weight_seed: int
    prompt_seed: int


TINY = ModelShape("tiny", 2, 256, 4, 4, 64, 1024, 4096, F16)
M2B = ModelShape("2b", 28, 2048, 16, 4, 128, 8192, 32000, F16)
M8B = ModelShape("8b", 32, 4096, 32, 8, 128, 14336, 128256, BF16)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, 16, 32, 1, 2),
    "2b": Workload("2b", M2B, 512, 1024, 5, 6),
    "2b_long": Workload("2b_long", M2B, 8192, 512, 5, 7),
    "8b": Workload("8b", M8B, 1024, 512, 8, 9),
}

# Isolated GEMV probe: two fp16 matrices, 1000 fresh vectors each.
GEMV_SHAPES = ((2048, 8192), (8192, 2048))
GEMV_SEEDS = (3, 4)
GEMV_N_VEC = 1000

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def layer_shapes(s: ModelShape) -> Dict[str, tuple]:
    qd = s.n_heads * s.head_dim
    kvd = s.n_kv_heads * s.head_dim
    return {
        "attn_norm": (s.d_model,),
        "wq": (qd, s.d_model),
        "wk": (kvd, s.d_model),
        "wv": (kvd, s.d_model),
        "wo": (s.d_model, qd),
        "ffn_norm": (s.d_model,),
        "w_gate": (s.d_ffn, s.d_model),
        "w_up": (s.d_ffn, s.d_model),
        "w_down": (s.d_model, s.d_ffn),
    }


def make_weights(s: ModelShape, seed: int, device="cpu", gain_jitter: float = 0.0,
                 std: float = 0.02) -> Dict[str, object]:
    """Weights of shape ``s`` in storage dtype on ``device``.

    Returns {"tok_emb", "final_norm", "lm_head", "layers": [dict per layer]}.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    dt = s.torch_dtype

    def mat(shape):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(dt)

    def gain(n):
        if gain_jitter > 0:
            r = torch.randn((n,), generator=g, device=dev, dtype=torch.float32)
            return (1.0 + gain_jitter * r).to(dt)
        return torch.ones((n,), device=dev, dtype=dt)

    w: Dict[str, object] = {"tok_emb": mat((s.vocab, s.d_model))}
    layers: List[Dict[str, torch.Tensor]] = []
    shapes = layer_shapes(s)
    for _ in range(s.n_layers):
        lw = {}
        for k in LAYER_KEYS:
            lw[k] = gain(shapes[k][0]) if k.endswith("norm") else mat(shapes[k])
        layers.append(lw)
    w["layers"] = layers
    w["final_norm"] = gain(s.d_model)
    w["lm_head"] = mat((s.vocab, s.d_model))
    return w


def weights_to(w: Dict[str, object], device) -> Dict[str, object]:
    out = {k: v.to(device) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: v.to(device) for k, v in lw.items()} for lw in w["layers"]]
    return out


def make_prompt(s: ModelShape, n: int, seed: int) -> torch.Tensor:
    g = torch.Generator()
    g.manual_seed(seed)
    return torch.randint(0, s.vocab, (n,), generator=g, dtype=torch.int64).to(torch.int32)


def make_kv(s: ModelShape, n_pos: int, seed: int, device="cpu", std: float = 1.0):
    """Synthetic KV cache (K, V) each [n_layers][Hkv][n_pos][hd] in storage dtype."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    shape = (s.n_layers, s.n_kv_heads, n_pos, s.head_dim)
    k = (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(s.torch_dtype)
    v = (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(s.torch_dtype)
    return k, v


def make_gemv(rows: int, cols: int, n_vec: int, seed: int, n_copies: int = 1, device="cpu",
              dtype=torch.float16, integer: bool = False):
    """GEMV probe inputs: W [n_copies][rows][cols] ~ N(0, 0.02^2) and x [n_vec][cols] ~ N(0, 1).

    With ``integer`` the entries are small integers (W in {-2..2}, x in {-2..2}) so
    every product and partial sum is exact in fp32 for cols <= 2^20 / 4.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if integer:
        W = torch.randint(-2, 3, (n_copies, rows, cols), generator=g, device=dev).to(dtype)
        x = torch.randint(-2, 3, (n_vec, cols), generator=g, device=dev).to(dtype)
    else:
        W = (torch.randn((n_copies, rows, cols), generator=g, device=dev) * 0.02).to(dtype)
        x = torch.randn((n_vec, cols), generator=g, device=dev).to(dtype)
    return W, x


def shape_by_name(name: str) -> ModelShape:
    return {"tiny": TINY, "2b": M2B, "8b": M8B}[name]


def param_count(s: ModelShape) -> int:
    per_layer = sum(int(torch.Size(v).numel()) for v in layer_shapes(s).values())
    return s.n_layers * per_layer + 2 * s.vocab * s.d_model + s.d_model


def small_shape(name="mini", n_layers=2, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16,
                d_ffn=128, vocab=97, dtype=F16) -> ModelShape:
    """A very small shape for CPU-only oracle tests."""
    return ModelShape(name, n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, dtype)


__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "TINY", "M2B", "M8B", "GEMV_SHAPES", "GEMV_SEEDS",
    "GEMV_N_VEC", "LAYER_KEYS", "layer_shapes", "make_weights", "weights_to", "make_prompt",
    "make_kv", "make_gemv", "shape_by_name", "param_count", "small_shape", "F16", "BF16",
]
