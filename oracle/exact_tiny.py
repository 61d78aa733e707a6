"""Exact-arithmetic definition of the row normalizations, for tiny rows.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is a second, independent statement of the same definitions as
``oracle.c``, used to pin the fp64 oracle: sums, means and variances are
exact rationals (``fractions.Fraction``), and the one square root is taken
with ``decimal`` at 60 significant digits, so each returned value is the true
result correctly rounded to a double (up to the 1e-60 relative error of the
root).

Definitions followed:
  - RMSNorm (Emily.Fast docs, `rms_norm`; Emily notebook, Part 1 composed
    cell): y_j = x_j / sqrt(mean_j(x_j^2) + eps) * w_j.
  - RMSNorm with the SiLU gate (mlx-c-rust `compile/norm_fusion.rs`, the
    output norm's SwiGLU epilogue, read as y_j = RMSNorm(x, w)_j * g_j /
    (1 + exp(-g_j))): the exponential taken with `decimal` at 60 digits.
  - LayerNorm (Emily.Fast docs, `layer_norm`): mean and (population) variance
    of the row, y_j = (x_j - mean) / sqrt(var + eps) * w_j + b_j.

Inputs are sequences of Python floats (every fp32 and bf16 value is an exact
double) and eps is the exact double value of the fp32 the kernels receive.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction
from typing import Sequence

_DIGITS = 60


def _to_decimal(q: Fraction) -> Decimal:
    return Decimal(q.numerator) / Decimal(q.denominator)


def _inv_sqrt(q: Fraction) -> Decimal:
    """1 / sqrt(q) for a rational q > 0, to _DIGITS digits."""
    return Decimal(1) / _to_decimal(q).sqrt()


def rms_row(x: Sequence[float], w: Sequence[float], eps: float) -> list[float]:
    n = len(x)
    xs = [Fraction(v) for v in x]
    mean_sq = sum(v * v for v in xs) / n
    denom_sq = mean_sq + Fraction(eps)
    with localcontext() as ctx:
        ctx.prec = _DIGITS
        if denom_sq == 0:
            # 0/0: the IEEE result of the definition is NaN for every element.
            return [float("nan")] * n
        s = _inv_sqrt(denom_sq)
        return [float(_to_decimal(xv * Fraction(wv)) * s) for xv, wv in zip(xs, w)]


def layer_row(x: Sequence[float], w: Sequence[float], b: Sequence[float] | None,
              eps: float) -> list[float]:
    n = len(x)
    xs = [Fraction(v) for v in x]
    mean = sum(xs) / n
    var = sum((v - mean) ** 2 for v in xs) / n
    denom_sq = var + Fraction(eps)
    bias = [Fraction(0)] * n if b is None else [Fraction(v) for v in b]
    with localcontext() as ctx:
        ctx.prec = _DIGITS
        if denom_sq == 0:
            return [float("nan")] * n
        s = _inv_sqrt(denom_sq)
        out = []
        for xv, wv, bv in zip(xs, w, bias):
            val = _to_decimal((xv - mean) * Fraction(wv)) * s + _to_decimal(bv)
            out.append(float(val))
        return out


def rms_swiglu_row(x: Sequence[float], g: Sequence[float], w: Sequence[float],
                   eps: float) -> list[float]:
    """RMSNorm of the row times SiLU of the gate, each value the true result
    rounded once to a double (up to the 60-digit working precision)."""
    n = len(x)
    xs = [Fraction(v) for v in x]
    denom_sq = sum(v * v for v in xs) / n + Fraction(eps)
    with localcontext() as ctx:
        ctx.prec = _DIGITS
        if denom_sq == 0:
            return [float("nan")] * n
        s = _inv_sqrt(denom_sq)
        out = []
        for xv, gv, wv in zip(xs, g, w):
            gd = Decimal(gv)                      # exact: a double is a finite decimal
            silu = gd / (Decimal(1) + (-gd).exp())
            out.append(float(_to_decimal(xv * Fraction(wv)) * s * silu))
        return out


def rms(rows: Sequence[Sequence[float]], w, eps) -> list[list[float]]:
    return [rms_row(r, w, eps) for r in rows]


def layer(rows: Sequence[Sequence[float]], w, b, eps) -> list[list[float]]:
    return [layer_row(r, w, b, eps) for r in rows]


def rope_row_complex(x, pos, dims, traditional, base, scale, freqs=None):
    """Rotary embedding of one head vector written as complex multiplication:
    pair i is the complex number z_i = x_a + 1j * x_b (a, b the pair's
    indices: (i, i + dims/2) split-half, (2i, 2i + 1) interleaved), and
    the result is z_i * exp(1j * theta_i) with theta_i = pos * scale *
    inv_freq_i, inv_freq_i = base ** (-2 i / dims) or freqs[i] (Emily.Fast
    docs, `rope` and `rope_with_freqs`).  Features past `dims` pass through.
    Plain Python floats and cmath."""
    import cmath

    out = list(x)
    half = dims // 2
    for i in range(half):
        inv = float(freqs[i]) if freqs is not None else float(base) ** (-2.0 * i / dims)
        theta = pos * float(scale) * inv
        a, b = (2 * i, 2 * i + 1) if traditional else (i, i + half)
        z = complex(x[a], x[b]) * cmath.exp(1j * theta)
        out[a], out[b] = z.real, z.imag
    return out
