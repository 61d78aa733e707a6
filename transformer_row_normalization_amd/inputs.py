"""Seeded synthetic inputs for the row-normalization workloads.

This module only draws random numbers and lays them out; it holds none of the
normalization arithmetic.  Both the HIP path and the CPU oracle are fed from
the tensors it returns (host tensors; callers copy them to the device).

Every tensor is drawn in fp32 from a CPU ``torch.Generator`` seeded per
workload, scaled and shifted in fp32, and, for bf16 workloads, cast to bf16
once (round to nearest even).

Workloads (name: shape, distribution):
  rms_f32_512x1024      x [4,128,1024] ~ U[-1,1), w = 1, eps 1e-6; the
                        variant ``iota`` sets x = fl32(i) / 100 over the
                        flattened index i, the input of the Emily notebook's
                        Part 1 correctness cell.
  layer_f32_1024x768    x [1,1024,768] ~ U[-1,1), w ~ U[0.5,1.5),
                        b ~ U[-0.1,0.1), eps 1e-6 (the LayerNorm A/B shape of
                        ffai-argus `examples/kernel_micro_ab.rs`).
  dual_bf16_4096tok     q [4096,32,128], k [4096,8,128] ~ N(0,1),
                        q_w, k_w [128] ~ N(1,0.1), eps 1e-6.
  rms_bf16_16384x8192   x [16384,8192] ~ N(0,1), w ~ N(1,0.1), eps 1e-5.
  layer_bf16_65536x4096 x [65536,4096] ~ N(3,1) with a Bernoulli(0.001) mask
                        of entries multiplied by 100, w ~ N(1,0.1),
                        b ~ N(0,0.02), eps 1e-5.
  rms_swiglu_bf16_4096tok  the gated output norm of a gated-delta block at
                        the dual workload's head layout: x [4096,32,128]
                        ~ N(0,1), gate g [4096,32,128] ~ N(0,2),
                        w [128] ~ N(1,0.1), eps 1e-6.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass
class Workload:
    name: str
    op: str                      # "rms" | "layer" | "dual" | "swiglu"
    dtype: torch.dtype
    eps: float
    tensors: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        if self.op == "dual":
            hd = self.tensors["q"].shape[-1]
            return (self.tensors["q"].numel() + self.tensors["k"].numel()) // hd
        x = self.tensors["x"]
        return x.numel() // x.shape[-1]

    @property
    def width(self) -> int:
        t = self.tensors["q"] if self.op == "dual" else self.tensors["x"]
        return t.shape[-1]


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(seed)


def uniform(shape, lo: float, hi: float, g: torch.Generator) -> torch.Tensor:
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def normal(shape, mean: float, std: float, g: torch.Generator) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32) * std + mean


def with_outliers(x: torch.Tensor, p: float, factor: float, g: torch.Generator):
    """Multiply a Bernoulli(p) subset of entries by ``factor``; returns
    (tensor, number of entries hit)."""
    mask = torch.rand(x.shape, generator=g, dtype=torch.float32) < p
    return torch.where(mask, x * factor, x), int(mask.sum())


def iota_over_100(shape) -> torch.Tensor:
    n = 1
    for s in shape:
        n *= s
    return (torch.arange(n, dtype=torch.float32) / 100.0).reshape(shape)


def rms_f32_512x1024(variant: str = "uniform") -> Workload:
    g = _gen(0)
    shape = (4, 128, 1024)
    if variant == "uniform":
        x = uniform(shape, -1.0, 1.0, g)
    elif variant == "iota":
        x = iota_over_100(shape)
    else:
        raise ValueError(variant)
    w = torch.ones(1024, dtype=torch.float32)
    return Workload(f"rms_f32_512x1024_{variant}", "rms", torch.float32, 1e-6, {"x": x, "w": w})


def layer_f32_1024x768() -> Workload:
    g = _gen(1)
    x = uniform((1, 1024, 768), -1.0, 1.0, g)
    w = uniform((768,), 0.5, 1.5, g)
    b = uniform((768,), -0.1, 0.1, g)
    return Workload("layer_f32_1024x768", "layer", torch.float32, 1e-6, {"x": x, "w": w, "b": b})


def dual_bf16_4096tok(tokens: int = 4096, q_heads: int = 32, k_heads: int = 8,
                      head_dim: int = 128) -> Workload:
    g = _gen(2)
    q = normal((tokens, q_heads, head_dim), 0.0, 1.0, g).to(torch.bfloat16)
    k = normal((tokens, k_heads, head_dim), 0.0, 1.0, g).to(torch.bfloat16)
    qw = normal((head_dim,), 1.0, 0.1, g).to(torch.bfloat16)
    kw = normal((head_dim,), 1.0, 0.1, g).to(torch.bfloat16)
    return Workload(f"dual_bf16_{tokens}tok", "dual", torch.bfloat16, 1e-6,
                    {"q": q, "k": k, "qw": qw, "kw": kw})


def rms_bf16_16384x8192(rows: int = 16384, width: int = 8192) -> Workload:
    g = _gen(3)
    x = normal((rows, width), 0.0, 1.0, g).to(torch.bfloat16)
    w = normal((width,), 1.0, 0.1, g).to(torch.bfloat16)
    return Workload(f"rms_bf16_{rows}x{width}", "rms", torch.bfloat16, 1e-5, {"x": x, "w": w})


def layer_bf16_65536x4096(rows: int = 65536, width: int = 4096) -> Workload:
    g = _gen(4)
    x = normal((rows, width), 3.0, 1.0, g)
    x, hits = with_outliers(x, 0.001, 100.0, g)
    x = x.to(torch.bfloat16)
    w = normal((width,), 1.0, 0.1, g).to(torch.bfloat16)
    b = normal((width,), 0.0, 0.02, g).to(torch.bfloat16)
    wl = Workload(f"layer_bf16_{rows}x{width}", "layer", torch.bfloat16, 1e-5,
                  {"x": x, "w": w, "b": b})
    wl.tensors["outliers"] = hits
    return wl


def rms_swiglu_bf16_4096tok(tokens: int = 4096, heads: int = 32,
                            head_dim: int = 128) -> Workload:
    g = _gen(5)
    x = normal((tokens, heads, head_dim), 0.0, 1.0, g).to(torch.bfloat16)
    gate = normal((tokens, heads, head_dim), 0.0, 2.0, g).to(torch.bfloat16)
    w = normal((head_dim,), 1.0, 0.1, g).to(torch.bfloat16)
    return Workload(f"rms_swiglu_bf16_{tokens}tok", "swiglu", torch.bfloat16, 1e-6,
                    {"x": x, "g": gate, "w": w})


def random_rows(op: str, rows: int, width: int, dtype: torch.dtype, seed: int,
                mean: float = 0.0, std: float = 1.0, with_bias: bool = True) -> dict:
    """Generic seeded inputs of any shape, for sweeps: x ~ N(mean, std),
    w ~ N(1, 0.1), b ~ N(0, 0.02) (LayerNorm), gate g ~ N(0, 3) (op
    "swiglu")."""
    g = _gen(seed)
    out = {"x": normal((rows, width), mean, std, g).to(dtype),
           "w": normal((width,), 1.0, 0.1, g).to(dtype)}
    if op == "layer" and with_bias:
        out["b"] = normal((width,), 0.0, 0.02, g).to(dtype)
    if op == "swiglu":
        out["g"] = normal((rows, width), 0.0, 3.0, g).to(dtype)
    return out


def large_rows_on_device(rows: int, width: int, dtype: torch.dtype, seed: int, device,
                         mean: float = 0.0, std: float = 1.0) -> dict:
    """Rows too large to build on the host (past 2^31 elements): x ~ N(mean,
    std) drawn by the device's seeded generator in fp32 slabs, cast once;
    w ~ N(1, 0.1) and b ~ N(0, 0.02) from the CPU generator.  Returns device
    tensors; callers copy sampled rows back for the oracle."""
    gdev = torch.Generator(device=device).manual_seed(seed)
    x = torch.empty((rows, width), dtype=dtype, device=device)
    slab = max(1, (1 << 27) // width)
    for r0 in range(0, rows, slab):
        n = min(slab, rows - r0)
        x[r0:r0 + n] = (torch.randn((n, width), generator=gdev, device=device,
                                    dtype=torch.float32) * std + mean).to(dtype)
    g = _gen(seed)
    return {"x": x, "w": normal((width,), 1.0, 0.1, g).to(dtype).to(device),
            "b": normal((width,), 0.0, 0.02, g).to(dtype).to(device)}


ALL = {
    "rms_f32_512x1024": rms_f32_512x1024,
    "layer_f32_1024x768": layer_f32_1024x768,
    "dual_bf16_4096tok": dual_bf16_4096tok,
    "rms_bf16_16384x8192": rms_bf16_16384x8192,
    "layer_bf16_65536x4096": layer_bf16_65536x4096,
    "rms_swiglu_bf16_4096tok": rms_swiglu_bf16_4096tok,
}
