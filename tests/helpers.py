"""Comparison helpers for the tests: dtype views, bf16 rounding of fp64
reference values, ulp distance and the tolerance checks.

Tolerances (fp32: relative error <= 1e-5; bf16: <= 1 ulp and <= 7.9e-3
relative; fp16: <= 1 ulp and <= 2^-10 relative, the relative error floored
at fp16's smallest normal 2^-14 where its spacing becomes absolute):
  RMSNorm      |y - r| / |r|                 (0/0 counts as 0)
  LayerNorm    |y - r| / max(|r|, |w_j|)     (a floor at the scale of one
                                              normalized entry, since
                                              (x - mean) * s * w + b can cancel)
  bf16 also    ulp distance between y and RNE_bf16(r) <= 1 (for LayerNorm
               where |r| >= |w_j|)
  RoPE outputs a rotated pair (a, b) can cancel too: the floor of both
               features is max(|w_a|, |w_b|), the scale of a normalized pair
"""
from __future__ import annotations

import numpy as np
import torch

F32_REL_TOL = 1e-5
BF16_REL_TOL = 2.0 ** -7      # 7.8125e-3 <= 7.9e-3
BF16_MAX_ULP = 1
F16_REL_TOL = 2.0 ** -10      # one fp16 ulp, relative, at worst
F16_MAX_ULP = 1
F16_MIN_NORMAL = 2.0 ** -14


def to_oracle_array(t: torch.Tensor) -> np.ndarray:
    """Host numpy view the oracle takes: float32, uint16 bf16 bits, or float16."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float32, torch.float16):
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def widen(t: torch.Tensor) -> np.ndarray:
    """A float32 or bf16 tensor as exact float64 numpy values."""
    return t.detach().cpu().to(torch.float64).numpy()


def rne_bf16_bits(r: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even)
    directly, without passing through float32; returns uint16 bit patterns."""
    r = np.asarray(r, dtype=np.float64)
    out = np.zeros(r.shape, dtype=np.float64)
    finite = np.isfinite(r) & (r != 0)
    m, e = np.frexp(r[finite])                # r = m * 2^e, 0.5 <= |m| < 1
    # bf16 has 8 significant bits; its smallest quantum is 2^-133.
    q_exp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, q_exp)
    out[finite] = np.rint(r[finite] / q) * q   # division by 2^k is exact
    out[~finite] = r[~finite]
    out32 = out.astype(np.float32)             # exact: out has <= 8 bits
    bits = out32.view(np.uint32) >> 16
    return bits.astype(np.uint16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return to_oracle_array(t.to(torch.bfloat16) if t.dtype != torch.bfloat16 else t)


def _ordered(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers ordered like the values."""
    b = bits.astype(np.int32)
    neg = (b & 0x8000) != 0
    return np.where(neg, -(b & 0x7FFF), b & 0x7FFF)


def ulp_distance_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(_ordered(a_bits) - _ordered(b_bits))


def f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def rne_f16_bits(r: np.ndarray) -> np.ndarray:
    """float64 values rounded to IEEE binary16 (numpy rounds directly from
    double, to nearest even); uint16 bit patterns."""
    with np.errstate(over="ignore"):
        return np.asarray(r, dtype=np.float64).astype(np.float16).view(np.uint16)


def rel_err(y: np.ndarray, r: np.ndarray, floor: np.ndarray | None = None) -> np.ndarray:
    """|y - r| / max(|r|, floor), with 0/0 := 0 and matching NaNs := 0."""
    denom = np.abs(r) if floor is None else np.maximum(np.abs(r), np.abs(floor))
    diff = np.abs(y - r)
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.where(diff == 0, 0.0, diff / denom)
    both_nan = np.isnan(y) & np.isnan(r)
    return np.where(both_nan, 0.0, e)


def check(op: str, y: torch.Tensor, r: np.ndarray, w: torch.Tensor | None = None,
          label: str = "", floor: np.ndarray | None = None) -> dict:
    """Assert the tolerance for one output tensor against the fp64 oracle.
    `floor` (broadcast to r's shape) replaces |w_j| as the error floor where
    the output can cancel (LayerNorm, rotations).  Returns the measured
    error figures."""
    yd = widen(y).reshape(r.shape)
    if floor is not None:
        floor = np.broadcast_to(np.abs(floor), r.shape)
    elif op == "layer":
        floor = np.broadcast_to(widen(w), r.shape)
    err = rel_err(yd, r, floor)
    nan_mismatch = int(np.sum(np.isnan(yd) != np.isnan(r)))
    out = {"max_rel": float(np.max(err)) if err.size else 0.0,
           "max_abs": float(np.nanmax(np.abs(yd - r))) if err.size else 0.0,
           "nan_mismatch": nan_mismatch}
    assert nan_mismatch == 0, f"{label}: NaN positions differ ({nan_mismatch})"
    if y.dtype == torch.float32:
        assert out["max_rel"] <= F32_REL_TOL, f"{label}: fp32 rel err {out['max_rel']:.3e}"
    elif y.dtype == torch.float16:
        # below the smallest normal (2^-14) fp16 has a fixed absolute spacing,
        # so relative error is measured against that floor; the ulp check
        # below covers the subnormal range exactly
        f16_floor = np.full(r.shape, F16_MIN_NORMAL) if floor is None else np.maximum(
            np.abs(floor), F16_MIN_NORMAL)
        out["max_rel"] = float(np.max(rel_err(yd, r, f16_floor))) if r.size else 0.0
        assert out["max_rel"] <= F16_REL_TOL, f"{label}: fp16 rel err {out['max_rel']:.3e}"
        ulps = ulp_distance_bf16(f16_bits(y).reshape(r.shape), rne_f16_bits(r))
        if floor is not None:
            ulps = np.where(np.abs(r) >= np.abs(floor), ulps, 0)
        ulps = np.where(np.isfinite(r), ulps, 0)
        out["max_ulp"] = int(ulps.max()) if ulps.size else 0
        assert out["max_ulp"] <= F16_MAX_ULP, f"{label}: fp16 ulp distance {out['max_ulp']}"
    else:
        assert out["max_rel"] <= BF16_REL_TOL, f"{label}: bf16 rel err {out['max_rel']:.3e}"
        ulps = ulp_distance_bf16(bf16_bits(y).reshape(r.shape), rne_bf16_bits(r))
        if floor is not None:
            mask = np.abs(r) >= np.abs(floor)
            ulps = np.where(mask, ulps, 0)
        finite = np.isfinite(r)
        ulps = np.where(finite, ulps, 0)
        out["max_ulp"] = int(ulps.max()) if ulps.size else 0
        assert out["max_ulp"] <= BF16_MAX_ULP, f"{label}: bf16 ulp distance {out['max_ulp']}"
    return out
