"""Comparison helpers for the tests: dtype views, rounding of fp64 reference
values, ulp distances and the tolerance checks.

Tolerances.  RMSNorm has no cancellation: its fp32 result carries a small
relative error, so it is checked pointwise everywhere:
  fp32   |y - r| / |r| <= 1e-5                       (0/0 counts as 0)
  bf16   ulp distance to RNE_bf16(r) <= 1, and |y - r| / |r| <= 2^-7
  fp16   ulp distance to RNE_f16(r) <= 1, and relative error <= 2^-10
         (floored at 2^-14, fp16's smallest normal)

LayerNorm and the rotated (RoPE) outputs can cancel: (x - mean) s w + b, or
a' cos - b' sin, can be far smaller than its terms, so a pure relative error
is not a property any fp32 evaluation has.  For these every output j gets an
absolute bound E_j on the error of the fp32 evaluation, derived from the
arithmetic (u = 2^-24, D = the longest chain of fp32 additions in the row
sums of any kernel able to serve the width, taken from the kernel names):

  LayerNorm  E_j = u ((D/2 + 8) |t_j| + (D + 2) k |w_j| + 2 |r_j|)
             t_j = (x_j - mean) s w_j = r_j - b_j, k = mean|x - mean| s <= 1
             per row for the kernels (corrected two-pass), k = mean|x| s for
             the composed chain
  RoPE       E_j = (|a_j| + |p_j|) (u (D/2 + 8) + T) + u |r_j|
             a_j, p_j the normalized values of the feature and its pair
             partner before the rotation, T the sine/cosine error

(derivation in layer_bound and rope_bound).  Then:
  fp32   |y - r| <= max(E_j, 1e-5 |r_j|) for every output
  bf16   ulp distance <= 1 wherever 2^-10 |r_j| >= E_j (there the fp32 value
         cannot cross two rounding boundaries: half an ulp of bf16 around
         r_j is at least 2^-10 |r_j|); elsewhere |y - r| <= E_j (1 + 2^-8)
         + 2^-8 |r_j| (the bound plus the final rounding); relative error
         <= 2^-7 against max(|r_j|, 2^10 E_j)
  fp16   the same with 2^-13 (and fp16's absolute half spacing 2^-25), the
         relative error against max(|r_j|, 2^13 E_j, 2^-14)
Each check returns its ulp histograms (all outputs, and those under the
ulp rule) so the tests can report them.
"""
from __future__ import annotations

import json
import math
import os
import re

import numpy as np
import torch

U32 = 2.0 ** -24              # unit roundoff of fp32
F32_REL_TOL = 1e-5
BF16_REL_TOL = 2.0 ** -7      # 7.8125e-3 <= 7.9e-3
BF16_MAX_ULP = 1
F16_REL_TOL = 2.0 ** -10      # one fp16 ulp, relative, at worst
F16_MAX_ULP = 1
F16_MIN_NORMAL = 2.0 ** -14

# Hardware sine / cosine error (v_sin_f32, v_cos_f32, argument in turns):
# the largest absolute error over every fp32 argument in [-1/2, 1/2] turns
# is 1.254e-7 (tests/hw_accuracy/trig_rsq.hip, run by test_hw_accuracy_gpu);
# the argument itself is an fp32 rounding of the fp64 fraction of a turn,
# at most 2^-26 turn = 9.37e-8 rad off.  v_rsq_f32's largest relative error
# is 9.4e-8 (< 2u), inside the 2u the bounds below allow for it.
HW_TRIG_ABS_ERR = 1.26e-7
HW_RSQ_REL_ERR = 9.5e-8
TRIG_ARG_ERR = 2.0 * math.pi * 2.0 ** -26


def to_oracle_array(t: torch.Tensor) -> np.ndarray:
    """Host numpy view the oracle takes: float32, uint16 bf16 bits, or float16."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float32, torch.float16):
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def widen(t) -> np.ndarray:
    """A float32 / bf16 / fp16 tensor (or array) as exact float64 numpy values."""
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


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
    """Map 16-bit float bit patterns to integers ordered like the values."""
    b = bits.astype(np.int32)
    neg = (b & 0x8000) != 0
    return np.where(neg, -(b & 0x7FFF), b & 0x7FFF)


def ulp_distance_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(_ordered(a_bits) - _ordered(b_bits))


def ulp_distance_f32(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Ulp distance between fp32 values y and the fp32 rounding of r."""
    def ordered(v):
        b = np.asarray(v, dtype=np.float32).view(np.int32).astype(np.int64)
        return np.where(b < 0, -(b & 0x7FFFFFFF), b)
    with np.errstate(over="ignore", invalid="ignore"):
        return np.abs(ordered(y) - ordered(np.asarray(r, dtype=np.float64).astype(np.float32)))


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


# ---------------------------------------------------------------- error bounds
def kernel_depth(name: str, width: int) -> int:
    """Longest chain of fp32 additions in one row sum of the kernel `name`
    (an fnorm_describe / fnorm_describe_rope name): each thread adds its
    elements one after another (VPT * VEC, or for the wide kernel every
    BLOCK * VEC-th element of the row), then the lane butterfly adds
    log2(lanes per row within a wave) times, then the per-wave partials are
    added in wave order (waves per row - 1)."""
    vec = int(re.search(r"\.vec(\d+)\.", name).group(1))
    if ".wide." in name:
        block = int(re.search(r"\.blk(\d+)", name).group(1))
        per_thread = -(-width // (block * vec)) * vec
        lanes, waves = 64, block // 64
    else:
        vpt = int(re.search(r"\.vpt(\d+)\.", name).group(1))
        lpr = int(re.search(r"\.lpr(\d+)\.", name).group(1))
        per_thread = vpt * vec
        lanes, waves = min(lpr, 64), max(1, lpr // 64)
    return per_thread + int(math.log2(lanes)) + waves - 1


def depth_bound(op_code: int, dtype_code: int, width: int) -> int:
    """The largest kernel_depth over every kernel the library offers for
    (op, dtype, width), aligned or not: whichever of them ran, its row sums
    are no deeper."""
    import transformer_row_normalization_amd as trn
    ops = (trn.OP_LAYER, trn.OP_LAYER_NOBIAS) if op_code in (trn.OP_LAYER, trn.OP_LAYER_NOBIAS) \
        else (op_code,)
    d = 1
    for op in ops:
        for aligned in (True, False):
            for v in range(trn.variant_count(op, dtype_code, width, aligned)):
                d = max(d, kernel_depth(trn.describe(op, dtype_code, width, aligned, v), width))
    return d


def rope_depth_bound(dtype_code: int, head_dim: int, dims: int, traditional: bool) -> int:
    import transformer_row_normalization_amd as trn
    d = 1
    for aligned in (True, False):
        for v in range(trn.rope_variant_count(dtype_code, head_dim, dims, traditional, aligned)):
            d = max(d, kernel_depth(trn.describe_rope(dtype_code, head_dim, dims, traditional,
                                                      aligned, v), head_dim))
    return d


def composed_depth(width: int) -> int:
    """Row sums of the composed chain: one thread of 256 adds every 256-th
    group of VEC <= 4 elements, then an 8-level LDS tree."""
    return -(-width // 256) + 3 + 8


def layer_bound(r: np.ndarray, w, b, depth: int, kappa=None) -> np.ndarray:
    """Bound on |y32 - r| for LayerNorm evaluated in fp32 (y32: the kernel's
    fp32 value before the final rounding).

    With d = x - mean, s = 1/sqrt(var + eps), t = d s w and r = t + b:
      * row sums of D additions err by at most D u of the sum of their
        magnitudes;
      * s: var carries at most (D + 4) u relative error (its sum, the
        correction c * sum(d), the scaling and the + eps), the square root
        halves it, v_rsq_f32 adds under 2u:  |ds/s| <= (D/2 + 4) u;
      * the centred value: the corrected two-pass removes the fp32 mean's
        error up to the error of c = sum(d)/N, at most (D + 1) u mean|d|,
        plus one rounding of x - mean and one of (x - mean) - c; times s w
        that is (D + 1) u mean|d| s |w| + 2u |t|, and mean|d| s <= 1
        (mean|d| <= sqrt(var) <= 1/s): kappa = mean|d| s <= 1 per row, which
        is mean_j |t_j / w_j| of the exact outputs (the default);
      * d s, then fma(d s, w, b): u |t| + u |r|.
    In all: |y32 - r| <= u ((D/2 + 7) |t| + (D + 1) kappa |w| + |r|).  The
    form used adds one u to each term (2 |r| covers the composed chain's
    separate multiply and add; kappa = mean|x| s for its uncorrected mean)."""
    r = np.asarray(r, dtype=np.float64)
    wd = np.broadcast_to(np.abs(widen(w)), r.shape)
    bd = np.zeros(r.shape) if b is None else np.broadcast_to(widen(b), r.shape)
    t = np.abs(r - bd)
    if kappa is None:
        # mean |d| s over the row, from the exact outputs: t_j / w_j = d_j s
        nz = wd != 0
        with np.errstate(invalid="ignore", divide="ignore"):
            q = np.where(nz & np.isfinite(t), t / np.where(nz, wd, 1.0), 0.0)
        cnt = np.maximum(nz.sum(axis=-1, keepdims=True), 1)
        k = np.minimum(q.sum(axis=-1, keepdims=True) / cnt, 1.0)
    else:
        k = np.asarray(kappa, dtype=np.float64)
        if k.ndim == 1:
            k = k.reshape(-1, *([1] * (r.ndim - 1))) if r.ndim > 1 else k
    return U32 * ((depth / 2 + 8) * t + (depth + 2) * k * wd + 2 * np.abs(r))


def composed_kappa(x) -> np.ndarray:
    """Per-row mean|x| / sqrt(var): the centring error scale of the composed
    chain, whose fp32 mean is not corrected (rows of x, last axis)."""
    xd = widen(x).reshape(-1, np.shape(x)[-1])
    sd = xd.std(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        k = np.where(sd > 0, np.abs(xd).mean(axis=1) / sd, 0.0)
    return np.maximum(k, 1.0)


def rope_bound(r: np.ndarray, plain: np.ndarray, dims: int, traditional: bool, depth: int,
               max_turns: float = 0.0) -> np.ndarray:
    """Bound on |y32 - r| for the rotated outputs of the fused dual + RoPE.

    `plain` are the normalized head vectors before the rotation (the oracle's
    dual RMSNorm, fp64), r the rotated ones, [..., head_dim].  For the pair
    (a, p) of a feature the kernel forms a32 = fl(fl(x s) w) (relative error
    (D/2 + 4) u + 2u, as for RMSNorm) and a32 c - p32 s' with c, s' the
    hardware cosine and sine of an fp32 fraction of a turn: |dc|, |ds'| <= T
    = HW_TRIG_ABS_ERR + TRIG_ARG_ERR + (fp64 angle error, max_turns 2^-50
    turns), so
      |y32 - r| <= (|a| + |p|) (u (D/2 + 6) + T) + 2u (|a| + |p|) + u |r|.
    Features at or past `dims` pass through: |y32 - r| <= u (D/2 + 6) |a|."""
    plain = np.asarray(plain, dtype=np.float64)
    a = np.abs(plain)
    partner = a.copy()
    half = dims // 2
    idx = np.arange(dims)
    pidx = (idx ^ 1) if traditional else np.where(idx < half, idx + half, idx - half)
    partner[..., :dims] = a[..., pidx]
    partner[..., dims:] = 0.0
    trig = np.zeros(a.shape[-1])
    trig[:dims] = HW_TRIG_ABS_ERR + TRIG_ARG_ERR + 2 * math.pi * max_turns * 2.0 ** -50
    return (a + partner) * (U32 * (depth / 2 + 8) + trig) + U32 * np.abs(r)


# ---------------------------------------------------------------- checks
def _hist(ulps: np.ndarray) -> dict:
    ulps = np.asarray(ulps).reshape(-1)
    return {"0": int(np.sum(ulps == 0)), "1": int(np.sum(ulps == 1)),
            "2": int(np.sum(ulps == 2)), "3+": int(np.sum(ulps >= 3))}


def merge_stats(acc: dict | None, e: dict) -> dict:
    """Combine the figures of two check() calls (chunks of one tensor)."""
    if acc is None:
        return json.loads(json.dumps(e))
    for k, v in e.items():
        if k in ("max_rel", "max_abs", "max_ulp", "max_ulp_all", "max_bound_use"):
            acc[k] = max(acc.get(k, 0), v)
        elif k in ("hist_all", "hist_checked"):
            acc[k] = {h: acc[k][h] + v[h] for h in v}
        elif k in ("n", "n_checked", "nan_mismatch"):
            acc[k] = acc.get(k, 0) + v
    acc["frac_checked"] = acc["n_checked"] / max(1, acc["n"])
    return acc


def check(op: str, y: torch.Tensor, r: np.ndarray, w: torch.Tensor | None = None,
          label: str = "", floor: np.ndarray | None = None, *, b=None,
          depth: int | None = None, bound: np.ndarray | None = None, kappa=None) -> dict:
    """Assert the tolerance for one output tensor against the fp64 oracle.

    op "rms": pointwise relative error (and ulps) everywhere; `floor`, if
      given, floors the relative error's denominator (a gated output can be
      exactly 0).
    op "layer": the LayerNorm bound (layer_bound with w, b, depth, kappa);
    `bound` given: that per-output absolute bound (RoPE).
    Returns the measured figures, with ulp histograms."""
    yd = widen(y).reshape(r.shape)
    if op == "layer" and bound is None:
        assert w is not None and depth is not None, f"{label}: LayerNorm needs w and depth"
        bound = layer_bound(r, w, b, depth, kappa)
    nan_mismatch = int(np.sum(np.isnan(yd) != np.isnan(r)))
    assert nan_mismatch == 0, f"{label}: NaN positions differ ({nan_mismatch})"
    finite = np.isfinite(r)
    with np.errstate(invalid="ignore"):
        diff = np.where(finite, np.abs(yd - r), 0.0)
    out = {"n": int(r.size), "nan_mismatch": 0,
           "max_abs": float(diff.max()) if r.size else 0.0}

    if bound is None:
        return _check_relative(y, yd, r, finite, floor, label, out)

    bound = np.broadcast_to(np.asarray(bound, dtype=np.float64), r.shape)
    absr = np.abs(r)
    if y.dtype == torch.float32:
        # how much of the bound the fp32 outputs use
        with np.errstate(invalid="ignore", divide="ignore"):
            use = np.where(diff == 0, 0.0, diff / bound)
        out["max_bound_use"] = float(np.max(np.where(finite, use, 0.0))) if r.size else 0.0
        lim = np.maximum(bound, F32_REL_TOL * absr)
        bad = finite & (diff > lim)
        assert not bad.any(), (f"{label}: fp32 error above max(E, 1e-5 |r|) at "
                               f"{np.argwhere(bad)[:3].tolist()} (diff {diff[bad][:3]}, "
                               f"E {bound[bad][:3]}, r {r[bad][:3]})")
        out["max_rel"] = float(np.max(rel_err(yd, r, 1e5 * bound)[finite])) if r.size else 0.0
        ulps = np.where(finite, ulp_distance_f32(yd.astype(np.float32), r), 0)
        zone = finite & (F32_REL_TOL * absr >= bound)
        assert out["max_rel"] <= F32_REL_TOL, f"{label}: fp32 rel err {out['max_rel']:.3e}"
    else:
        bf = y.dtype == torch.bfloat16
        shift = 2.0 ** -10 if bf else 2.0 ** -13
        spacing = 0.0 if bf else 2.0 ** -25
        rnd = 2.0 ** -8 if bf else 2.0 ** -11
        if bf:
            ulps = ulp_distance_bf16(bf16_bits(y).reshape(r.shape), rne_bf16_bits(r))
        else:
            ulps = ulp_distance_bf16(f16_bits(y).reshape(r.shape), rne_f16_bits(r))
        ulps = np.where(finite, ulps, 0)
        zone = finite & (np.maximum(shift * absr, spacing) >= bound)
        worst = int(np.max(np.where(zone, ulps, 0))) if r.size else 0
        assert worst <= 1, (f"{label}: ulp distance {worst} where the bound allows 1 at "
                            f"{np.argwhere(zone & (ulps > 1))[:3].tolist()}")
        rest = finite & ~zone
        lim = bound * (1 + rnd) + rnd * absr + spacing
        bad = rest & (diff > lim)
        assert not bad.any(), (f"{label}: error above the bound where cancellation "
                               f"allows more than an ulp: diff {diff[bad][:3]}, "
                               f"E {bound[bad][:3]}, r {r[bad][:3]}")
        tol = BF16_REL_TOL if bf else F16_REL_TOL
        # as in the pointwise check: below fp16's smallest normal (2^-14) the
        # spacing is a fixed 2^-24, so relative error is taken against 2^-14
        # there (one subnormal step is 2^-10 of it); the ulp rule above
        # covers that range exactly
        rfloor = np.maximum(bound / shift, spacing * 2 if bf else F16_MIN_NORMAL)
        out["max_rel"] = float(np.max(rel_err(yd, r, rfloor)[finite])) if r.size else 0.0
        assert out["max_rel"] <= tol, f"{label}: rel err {out['max_rel']:.3e}"
        out["max_ulp"] = worst
    out["max_ulp_all"] = int(ulps.max()) if r.size else 0
    out["n_checked"] = int(zone.sum())
    out["frac_checked"] = out["n_checked"] / max(1, r.size)
    out["hist_all"] = _hist(ulps[finite])
    out["hist_checked"] = _hist(ulps[zone])
    return out


def _check_relative(y, yd, r, finite, floor, label, out):
    """Pointwise relative error (and ulp distance) for outputs without
    cancellation (RMSNorm and its forms)."""
    if floor is not None:
        floor = np.broadcast_to(np.abs(np.asarray(floor, dtype=np.float64)), r.shape)
    err = rel_err(yd, r, floor)
    out["max_rel"] = float(np.max(err)) if err.size else 0.0
    if y.dtype == torch.float32:
        assert out["max_rel"] <= F32_REL_TOL, f"{label}: fp32 rel err {out['max_rel']:.3e}"
        ulps = np.where(finite, ulp_distance_f32(yd.astype(np.float32), r), 0)
    elif y.dtype == torch.float16:
        # below the smallest normal (2^-14) fp16 has a fixed absolute spacing,
        # so relative error is measured against that floor; the ulp check
        # covers the subnormal range exactly
        f16_floor = np.full(r.shape, F16_MIN_NORMAL) if floor is None else np.maximum(
            floor, F16_MIN_NORMAL)
        out["max_rel"] = float(np.max(rel_err(yd, r, f16_floor))) if r.size else 0.0
        assert out["max_rel"] <= F16_REL_TOL, f"{label}: fp16 rel err {out['max_rel']:.3e}"
        ulps = np.where(finite, ulp_distance_bf16(f16_bits(y).reshape(r.shape),
                                                  rne_f16_bits(r)), 0)
        out["max_ulp"] = int(ulps.max()) if ulps.size else 0
        assert out["max_ulp"] <= F16_MAX_ULP, f"{label}: fp16 ulp distance {out['max_ulp']}"
    else:
        assert out["max_rel"] <= BF16_REL_TOL, f"{label}: bf16 rel err {out['max_rel']:.3e}"
        ulps = np.where(finite, ulp_distance_bf16(bf16_bits(y).reshape(r.shape),
                                                  rne_bf16_bits(r)), 0)
        out["max_ulp"] = int(ulps.max()) if ulps.size else 0
        assert out["max_ulp"] <= BF16_MAX_ULP, f"{label}: bf16 ulp distance {out['max_ulp']}"
    out["max_ulp_all"] = int(ulps.max()) if ulps.size else 0
    out["n_checked"] = int(finite.sum())
    out["frac_checked"] = out["n_checked"] / max(1, r.size)
    out["hist_all"] = _hist(ulps[finite])
    out["hist_checked"] = out["hist_all"]
    return out


_DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
_DEPTHS: dict = {}


def row_depth(op: str, dtype: torch.dtype, width: int) -> int:
    """depth_bound for a row op ("rms" or "layer"), cached."""
    key = (op, dtype, width)
    if key not in _DEPTHS:
        import transformer_row_normalization_amd as trn
        _DEPTHS[key] = depth_bound(trn.OP_RMS if op == "rms" else trn.OP_LAYER,
                                   _DTYPE_CODE[dtype], width)
    return _DEPTHS[key]


def check_row(op: str, y: torch.Tensor, r: np.ndarray, w=None, b=None, label: str = "",
              kappa=None, kernel: str | None = None) -> dict:
    """check() for the output of a fused row op: RMSNorm pointwise, LayerNorm
    against layer_bound with the depth of `kernel` (the name of the kernel
    that ran) or, without one, of every kernel serving its width."""
    if op == "rms":
        return check("rms", y, r, label=label)
    d = kernel_depth(kernel, r.shape[-1]) if kernel else row_depth("layer", y.dtype, r.shape[-1])
    return check("layer", y, r, w, label, b=b, depth=d, kappa=kappa)


def check_rope(o, q, k, qw, kw, yq, yk, rq, rk, dims: int, traditional: bool, label: str,
               max_turns: float = 0.0, eps: float = 1e-6) -> dict:
    """Check fused dual + RoPE outputs (host tensors) against rope_bound; the
    values before the rotation are the oracle's plain dual RMSNorm."""
    hd = q.shape[-1]
    d = rope_depth_bound(_DTYPE_CODE[q.dtype], hd, dims, traditional)
    pq, pk = o.dual_head_rms(*(to_oracle_array(t) for t in (q, k, qw, kw)), eps)
    out = {}
    if q.numel():
        out["q"] = check("rms", yq, rq, label=f"{label} q",
                         bound=rope_bound(rq, pq, dims, traditional, d, max_turns))
    if k.numel():
        out["k"] = check("rms", yk, rk, label=f"{label} k",
                         bound=rope_bound(rk, pk, dims, traditional, d, max_turns))
    return out


def report(name: str, stats: dict) -> None:
    """Record a check's figures: printed, and appended as one JSON line to
    the file named by FNORM_ULP_REPORT when that is set."""
    line = json.dumps({"case": name, **stats})
    print(f"[ulp] {line}", flush=True)
    path = os.environ.get("FNORM_ULP_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
