"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
mathematics, independent of the oracle's own code.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
is wrong.  ``tests/test_oracle.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` runs them on deliberately broken copies of
``oracle.c`` and requires every mutant to fail at least one pin.

What pins what:
  golden hand cases      the pages' doc-example inputs evaluated exactly
                         (tests/golden/hand_cases.json, exact rationals)
  exact brute force      random tiny rows (widths 1..16, fp32 and bf16
                         inputs, random weight/bias/eps) against
                         oracle/exact_tiny.py
  unit-RMS invariant     w = 1:  mean(y^2) = ms / (ms + eps)
  LayerNorm moments      w = 1, b = 0:  mean(y) = 0, mean(y^2) = v / (v + eps)
  library identities     eps = 0: RMS = sqrt(N) x / ||x||_2 (numpy norm),
                         LayerNorm = population z-score (numpy mean/std)
  special cases          zero row, constant row, width 1, NaN propagation
  invariances            LayerNorm(x + c) = LayerNorm(x); RMS(a x) = RMS(x)
  affine structure       y(w, b) = y(1, 0) * w + b, column-indexed weights
  row independence       permuting rows permutes outputs, bitwise
  bf16 / f16 decoding    hand-built bf16 and binary16 bit patterns (normal,
                         subnormal, largest, inf, NaN) decode to the values
                         the formats define
  dual q/k               each half against exact brute force, queries first
  RoPE                   golden values of the `rope` / `rope_with_freqs` doc
                         inputs from a complex-number formulation
                         (oracle/exact_tiny.py), norm preservation, identity
                         at position 0, relative-position invariance,
                         composition of offsets, scale as a position
                         multiplier, interleaved = permuted split-half, an
                         exact inverse-frequency table = the schedule,
                         features past dims unchanged, dual + RoPE
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import exact_tiny

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "hand_cases.json")


def f32(v):
    return float(np.float32(v))


def _bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (RNE), numpy only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def _bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _close(a, b, rtol, floor=None, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = np.abs(b) if floor is None else np.maximum(np.abs(b), floor)
    err = np.abs(a - b)
    bad = err > rtol * scale
    bad &= ~(np.isnan(a) & np.isnan(b))
    assert not np.any(bad), f"{what}: max err {np.max(err):.3e} (rtol {rtol})"


# --------------------------------------------------------------------------
def pin_golden_hand_cases(o):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if c["op"] == "rope":
            fr = None if c["freqs"] is None else np.array(c["freqs"], np.float32)
            got = o.rope_rows(np.array(c["x"], np.float64), 1, c["dims"], c["traditional"],
                              c["base"], c["scale"], c["offset"], fr)
            _close(got, np.array(c["y"]), 1e-13, floor=1e-12, what=c["name"])
            continue
        x = np.array(c["x"], dtype=np.float32)
        w = np.array(c["w"], dtype=np.float32)
        exp = np.array(c["y"], dtype=np.float64)
        if c["op"] == "rms":
            got = o.rms(x, w, c["eps_f32"])
        else:
            got = o.layer(x, w, np.array(c["b"], dtype=np.float32), c["eps_f32"])
        _close(got, exp, 1e-14, floor=1e-300, what=c["name"])


def _tiny_rows(rng, dtype, width, rows):
    x = rng.standard_normal((rows, width)).astype(np.float32) * np.float32(rng.uniform(0.1, 5))
    x += np.float32(rng.uniform(-3, 3))
    w = rng.uniform(-2, 2, width).astype(np.float32)
    b = rng.uniform(-1, 1, width).astype(np.float32)
    if dtype == "bf16":
        xb, wb, bb = _bf16_from_f32(x), _bf16_from_f32(w), _bf16_from_f32(b)
        return (xb, wb, bb), (_bf16_values(xb), _bf16_values(wb), _bf16_values(bb))
    if dtype == "f16":
        xh, wh, bh = x.astype(np.float16), w.astype(np.float16), b.astype(np.float16)
        return (xh, wh, bh), (xh.astype(np.float64), wh.astype(np.float64), bh.astype(np.float64))
    return (x, w, b), (x.astype(np.float64), w.astype(np.float64), b.astype(np.float64))


def pin_exact_bruteforce_rms(o):
    rng = np.random.default_rng(101)
    for width in range(1, 17):
        for dtype in ("f32", "bf16", "f16"):
            (x, w, _), (xv, wv, _) = _tiny_rows(rng, dtype, width, 3)
            eps = f32(rng.choice([0.0, 1e-6, 1e-5, 0.5]))
            got = o.rms(x, w, eps)
            exp = np.array(exact_tiny.rms(xv.tolist(), wv.tolist(), eps))
            _close(got, exp, 1e-13, floor=1e-300, what=f"rms width {width} {dtype}")


def pin_exact_bruteforce_layer(o):
    rng = np.random.default_rng(202)
    for width in range(1, 17):
        for dtype in ("f32", "bf16", "f16"):
            for use_bias in (True, False):
                (x, w, b), (xv, wv, bv) = _tiny_rows(rng, dtype, width, 3)
                eps = f32(rng.choice([1e-6, 1e-5, 0.5]))
                got = o.layer(x, w, b if use_bias else None, eps)
                exp = np.array(exact_tiny.layer(xv.tolist(), wv.tolist(),
                                                bv.tolist() if use_bias else None, eps))
                floor = np.abs(wv) + (np.abs(bv) if use_bias else 0.0) + 1e-300
                _close(got, exp, 1e-13, floor=floor, what=f"layer width {width} {dtype}")


def pin_rms_unit_invariant(o):
    rng = np.random.default_rng(303)
    for eps in (0.3, 1e-6):
        x = rng.uniform(-1, 1, (8, 64)).astype(np.float32)
        y = o.rms(x, np.ones(64, np.float32), f32(eps))
        ms = np.mean(x.astype(np.float64) ** 2, axis=1)
        _close(np.mean(y ** 2, axis=1), ms / (ms + f32(eps)), 1e-12, what="unit RMS")


def pin_layer_moments(o):
    rng = np.random.default_rng(404)
    for eps in (0.3, 1e-5):
        x = (rng.standard_normal((8, 96)) * 2 + 5).astype(np.float32)
        y = o.layer(x, np.ones(96, np.float32), np.zeros(96, np.float32), f32(eps))
        v = np.var(x.astype(np.float64), axis=1)        # population variance
        assert np.max(np.abs(np.mean(y, axis=1))) < 1e-12, "LayerNorm mean not 0"
        _close(np.mean(y ** 2, axis=1), v / (v + f32(eps)), 1e-12, what="LN var")


def pin_library_identities(o):
    rng = np.random.default_rng(505)
    x = rng.uniform(-2, 2, (6, 50)).astype(np.float32)
    xd = x.astype(np.float64)
    ones = np.ones(50, np.float32)
    rms = o.rms(x, ones, 0.0)
    ref = xd * np.sqrt(50) / np.linalg.norm(xd, axis=1, keepdims=True)
    _close(rms, ref, 1e-13, what="RMS vs sqrt(N) x/||x||")
    ln = o.layer(x, ones, None, 0.0)
    z = (xd - xd.mean(axis=1, keepdims=True)) / xd.std(axis=1, keepdims=True)
    _close(ln, z, 1e-12, floor=1.0, what="LayerNorm vs z-score")


def pin_special_cases(o):
    w = np.array([1.5, -0.5, 2.0, 0.25], np.float32)
    b = np.array([0.1, 0.2, -0.3, 0.4], np.float32)
    # zero row, eps > 0: RMS gives exact zeros
    y = o.rms(np.zeros((1, 4), np.float32), w, f32(1e-6))
    assert np.all(y == 0.0), "RMS of zero row"
    # constant row: LayerNorm gives exactly the bias
    y = o.layer(np.full((2, 4), 3.25, np.float32), w, b, f32(1e-5))
    assert np.array_equal(y, np.broadcast_to(b.astype(np.float64), (2, 4))), "LN const row"
    # width 1
    x1 = np.array([[2.0], [-0.5]], np.float32)
    y = o.rms(x1, np.array([3.0], np.float32), 0.25)
    _close(y[:, 0], [2.0 / np.sqrt(4.25) * 3.0, -0.5 / np.sqrt(0.5) * 3.0], 1e-15, what="RMS w1")
    y = o.layer(x1, np.array([3.0], np.float32), np.array([0.75], np.float32), 0.25)
    assert np.all(y == 0.75), "LN width 1 gives the bias"
    # NaN in one row poisons only that row
    x = np.ones((3, 4), np.float32)
    x[1, 2] = np.nan
    for y in (o.rms(x, w, f32(1e-6)), o.layer(x, w, b, f32(1e-6))):
        assert np.all(np.isnan(y[1])) and np.all(np.isfinite(y[[0, 2]])), "NaN propagation"
    # zero row with eps = 0: 0/0 is NaN
    y = o.rms(np.zeros((1, 4), np.float32), w, 0.0)
    assert np.all(np.isnan(y)), "RMS 0/0"


def pin_invariances(o):
    rng = np.random.default_rng(606)
    # multiples of 2^-10 in [-4, 4): adding 7 and scaling by 4 stay exact in fp32
    x = (rng.integers(-4096, 4096, (5, 40)) / 1024.0).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 40).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 40).astype(np.float32)
    y0 = o.layer(x, w, b, f32(1e-5))
    y1 = o.layer(x + np.float32(7.0), w, b, f32(1e-5))
    _close(y1, y0, 1e-12, floor=1.0, what="LN shift invariance")
    r0 = o.rms(x, w, 0.0)
    r1 = o.rms(x * np.float32(4.0), w, 0.0)
    _close(r1, r0, 1e-14, floor=1e-300, what="RMS scale invariance")


def pin_affine_structure(o):
    rng = np.random.default_rng(707)
    x = rng.standard_normal((4, 12)).astype(np.float32)
    w = rng.uniform(-2, 2, 12).astype(np.float32)
    b = rng.uniform(-1, 1, 12).astype(np.float32)
    ones, zeros = np.ones(12, np.float32), np.zeros(12, np.float32)
    _close(o.rms(x, w, f32(1e-6)), o.rms(x, ones, f32(1e-6)) * w, 1e-15, floor=1e-300,
           what="RMS weight per column")
    base = o.layer(x, ones, zeros, f32(1e-6))
    _close(o.layer(x, w, b, f32(1e-6)), base * w + b, 1e-14, floor=1.0,
           what="LN weight and bias per column")
    # a NULL bias is the zero bias
    assert np.array_equal(o.layer(x, w, None, f32(1e-6)), o.layer(x, w, zeros, f32(1e-6)))


def pin_row_independence(o):
    rng = np.random.default_rng(808)
    x = rng.standard_normal((7, 33)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 33).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 33).astype(np.float32)
    perm = rng.permutation(7)
    assert np.array_equal(o.rms(x[perm], w, f32(1e-6)), o.rms(x, w, f32(1e-6))[perm])
    assert np.array_equal(o.layer(x[perm], w, b, f32(1e-6)), o.layer(x, w, b, f32(1e-6))[perm])


def pin_bf16_decoding(o):
    # sign | 8 exponent bits (bias 127) | 7 mantissa bits:
    # 0x3F80 = +1.0, 0x4000 = +2.0, 0xC040 = -3.0, 0x4090 = +4.5, 0x3E20 = 0.15625
    bits = np.array([[0x3F80, 0x4000, 0xC040, 0x4090, 0x3E20]], np.uint16)
    vals = [1.0, 2.0, -3.0, 4.5, 0.15625]
    wb = np.array([0x3F80, 0x3F00, 0x4000, 0xBF80, 0x3F80], np.uint16)   # 1, .5, 2, -1, 1
    wv = [1.0, 0.5, 2.0, -1.0, 1.0]
    got = o.rms(bits, wb, 0.0)
    _close(got[0], exact_tiny.rms_row(vals, wv, 0.0), 1e-15, what="bf16 decode (rms)")
    got = o.layer(bits, wb, wb, 0.0)
    _close(got[0], exact_tiny.layer_row(vals, wv, wv, 0.0), 1e-14, floor=1.0,
           what="bf16 decode (layer)")


def pin_f16_decoding(o):
    # binary16: sign | 5 exponent bits (bias 15) | 10 fraction bits
    # 0x3C00 = 1, 0xC000 = -2, 0x3555 = 0.333251953125, 0x7BFF = 65504 (largest),
    # 0x0400 = 2^-14 (smallest normal), 0x0001 = 2^-24 (smallest subnormal),
    # 0x8200 = -2^-15 (subnormal)
    bits = np.array([0x3C00, 0xC000, 0x3555, 0x7BFF, 0x0400, 0x0001, 0x8200], np.uint16)
    vals = [1.0, -2.0, 0.333251953125, 65504.0, 2.0 ** -14, 2.0 ** -24, -2.0 ** -15]
    ones = np.ones(1, np.float16)
    x = bits.view(np.float16).reshape(7, 1)
    got = o.rms(x, ones, 0.0)                    # width 1, eps 0: x / |x| = sign(x)
    assert np.array_equal(got[:, 0], np.sign(vals)), "f16 decode (sign)"
    # eps = 1: y = x / sqrt(x^2 + 1), invertible: x = y / sqrt(1 - y^2)
    got = o.rms(x, ones, 1.0)[:, 0]
    sel = [0, 1, 2, 4, 5, 6]
    back = got[sel] / np.sqrt(1.0 - got[sel] ** 2)
    _close(back, np.array(vals)[sel], 1e-12, what="f16 decode (values)")
    assert abs(got[3] - 65504.0 / np.sqrt(65504.0 ** 2 + 1)) < 1e-15
    inf = np.array([[0x7C00], [0xFC00], [0x7E00]], np.uint16).view(np.float16)
    r = o.rms(inf, ones, 1.0)[:, 0]
    assert np.isnan(r).all(), "f16 inf/nan decode (inf/inf and nan)"


def pin_dual(o):
    rng = np.random.default_rng(909)
    for dtype in ("f32", "bf16"):
        (q, qw, _), (qv, qwv, _) = _tiny_rows(rng, dtype, 8, 6)
        (k, kw, _), (kv, kwv, _) = _tiny_rows(rng, dtype, 8, 2)
        eps = f32(1e-6)
        qy, ky = o.dual_head_rms(q.reshape(3, 2, 8), k.reshape(1, 2, 8), qw, kw, eps)
        assert qy.shape == (3, 2, 8) and ky.shape == (1, 2, 8)
        _close(qy.reshape(6, 8), exact_tiny.rms(qv.tolist(), qwv.tolist(), eps), 1e-13,
               floor=1e-300, what=f"dual queries {dtype}")
        _close(ky.reshape(2, 8), exact_tiny.rms(kv.tolist(), kwv.tolist(), eps), 1e-13,
               floor=1e-300, what=f"dual keys {dtype}")


# ------------------------------------------------------------------ RoPE
def _rope_input(rng, rows, hd):
    return rng.standard_normal((rows, hd))


def pin_rope_norm_and_identity(o):
    rng = np.random.default_rng(1101)
    v = _rope_input(rng, 12, 16)
    for trad in (False, True):
        y = o.rope_rows(v, 3, 16, trad, 10000.0, 1.0, 5)
        _close(np.linalg.norm(y, axis=1), np.linalg.norm(v, axis=1), 1e-14, what="rope norm")
        y0 = o.rope_rows(v, 12, 16, trad, 10000.0, 1.0, 0)      # every row at position 0
        assert np.array_equal(y0, v), "rope at position 0 is the identity"
        # each rotated pair keeps its own length
        y = o.rope_rows(v, 1, 16, trad, 300.0, 1.0, 2)
        a = np.arange(8) * 2 if trad else np.arange(8)
        b = a + 1 if trad else a + 8
        _close(y[:, a] ** 2 + y[:, b] ** 2, v[:, a] ** 2 + v[:, b] ** 2, 1e-13,
               what="rope pair length")


def pin_rope_relative_position(o):
    # <rope(a, p), rope(b, p + k)> depends only on k
    rng = np.random.default_rng(1102)
    a, b = _rope_input(rng, 1, 32), _rope_input(rng, 1, 32)
    for trad in (False, True):
        ref = None
        for p in (0, 3, 100):
            ra = o.rope_rows(a, 1, 32, trad, 10000.0, 1.0, p)
            rb = o.rope_rows(b, 1, 32, trad, 10000.0, 1.0, p + 7)
            d = float((ra @ rb.T)[0, 0])
            ref = d if ref is None else ref
            assert abs(d - ref) < 1e-12 * (1 + abs(ref)), "rope relative position"


def pin_rope_composition_and_scale(o):
    rng = np.random.default_rng(1103)
    v = _rope_input(rng, 6, 16)
    for trad in (False, True):
        once = o.rope_rows(v, 6, 16, trad, 10000.0, 1.0, 9)      # one token: position = offset
        twice = o.rope_rows(o.rope_rows(v, 6, 16, trad, 10000.0, 1.0, 4), 6, 16, trad,
                            10000.0, 1.0, 5)
        _close(twice, once, 1e-13, floor=1e-12, what="rope composition")
        s2 = o.rope_rows(v, 6, 16, trad, 10000.0, 2.0, 9)
        p2 = o.rope_rows(v, 6, 16, trad, 10000.0, 1.0, 18)
        _close(s2, p2, 1e-13, floor=1e-12, what="rope scale multiplies the position")


def pin_rope_layouts_and_table(o):
    rng = np.random.default_rng(1104)
    v = _rope_input(rng, 8, 16)
    # interleaved pairs (2i, 2i+1) are the split-half pairs (i, i+8) after
    # gathering the even then the odd features
    perm = np.concatenate([np.arange(0, 16, 2), np.arange(1, 16, 2)])
    trad = o.rope_rows(v, 2, 16, True, 10000.0, 1.0, 3)
    split = o.rope_rows(v[:, perm], 2, 16, False, 10000.0, 1.0, 3)
    _close(split, trad[:, perm], 1e-14, floor=1e-12, what="rope layouts")
    # base 16 over 8 dims has inverse frequencies 16^(-2i/8) = 2^-i exactly
    table = np.array([1, .5, .25, .125], np.float32)
    for trad in (False, True):
        tab8 = o.rope_rows(v[:, :8], 2, 8, trad, 1.0, 1.0, 3, table)
        sch8 = o.rope_rows(v[:, :8], 2, 8, trad, 16.0, 1.0, 3)
        assert np.array_equal(tab8, sch8), "rope table equals the schedule"
    # features past dims pass through unchanged
    p = o.rope_rows(v, 2, 6, False, 10000.0, 1.0, 3)
    assert np.array_equal(p[:, 6:], v[:, 6:]), "rope tail"


def pin_dual_rope(o):
    rng = np.random.default_rng(1105)
    for dtype in ("f32", "bf16"):
        (q, qw, _), _ = _tiny_rows(rng, dtype, 16, 6)
        (k, kw, _), _ = _tiny_rows(rng, dtype, 16, 3)
        q3, k3 = q.reshape(3, 2, 16), k.reshape(3, 1, 16)
        plain_q, plain_k = o.dual_head_rms(q3, k3, qw, kw, f32(1e-6))
        for trad in (False, True):
            fq, fk = o.dual_head_rms_rope(q3, k3, qw, kw, f32(1e-6), 16, trad, 10000.0, 1.0, 0)
            # token 0 sits at position 0: unrotated
            assert np.array_equal(fq[0], plain_q[0]) and np.array_equal(fk[0], plain_k[0])
            # rotation keeps each head vector's length
            _close(np.linalg.norm(fq, axis=2), np.linalg.norm(plain_q, axis=2), 1e-13,
                   what="dual rope q norm")
            _close(np.linalg.norm(fk, axis=2), np.linalg.norm(plain_k, axis=2), 1e-13,
                   what="dual rope k norm")
            # the keys of token t rotate like a query head of token t
            fq2, fk2 = o.dual_head_rms_rope(q3, k3, qw, kw, f32(1e-6), 16, trad, 10000.0, 1.0, 4)
            rk = o.rope_rows(plain_k.reshape(3, 16), 1, 16, trad, 10000.0, 1.0, 4)
            _close(fk2.reshape(3, 16), rk, 1e-14, floor=1e-12, what="dual rope keys")


def _gate_like(rng, dtype, shape):
    """Gate values over the range where SiLU is neither 0 nor linear, plus
    a few saturated ones, in the element type of the test."""
    g = (rng.standard_normal(shape) * 4).astype(np.float32)
    g.flat[::7] = np.float32(rng.choice([-60.0, -25.0, 25.0, 60.0]))
    if dtype == "bf16":
        gb = _bf16_from_f32(g)
        return gb, _bf16_values(gb)
    if dtype == "f16":
        gh = g.astype(np.float16)
        return gh, gh.astype(np.float64)
    return g, g.astype(np.float64)


def pin_rms_swiglu_bruteforce(o):
    # exact-rational norm times a 60-digit SiLU, widths 1..16, all types
    rng = np.random.default_rng(1201)
    for width in range(1, 17):
        for dtype in ("f32", "bf16", "f16"):
            (x, w, _), (xv, wv, _) = _tiny_rows(rng, dtype, width, 2)
            g, gv = _gate_like(rng, dtype, x.shape)
            eps = f32(rng.choice([1e-6, 1e-5, 0.5]))
            got = o.rms_swiglu(x, g, w, eps)
            exp = np.array([exact_tiny.rms_swiglu_row(xr.tolist(), gr.tolist(), wv.tolist(), eps)
                            for xr, gr in zip(xv, gv)])
            _close(got, exp, 1e-13, floor=1e-300, what=f"rms_swiglu width {width} {dtype}")


def pin_rms_swiglu_gate_identities(o):
    rng = np.random.default_rng(1202)
    x = rng.standard_normal((5, 24)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 24).astype(np.float32)
    plain = o.rms(x, w, f32(1e-6))
    # SiLU(0) = 0: a zero gate closes the output exactly
    assert np.all(o.rms_swiglu(x, np.zeros_like(x), w, f32(1e-6)) == 0.0), "zero gate"
    # SiLU(g) - SiLU(-g) = g (since sigmoid(g) + sigmoid(-g) = 1)
    g = (rng.standard_normal(x.shape) * 3).astype(np.float32)
    diff = o.rms_swiglu(x, g, w, f32(1e-6)) - o.rms_swiglu(x, -g, w, f32(1e-6))
    _close(diff, plain * g.astype(np.float64), 1e-13, floor=1e-12, what="odd part of the gate")
    # the tanh form of the same gate: SiLU(g) = g/2 * (1 + tanh(g/2))
    gd = g.astype(np.float64)
    _close(o.rms_swiglu(x, g, w, f32(1e-6)), plain * gd / 2 * (1 + np.tanh(gd / 2)), 1e-13,
           floor=1e-12, what="tanh form")
    # a large gate passes through: SiLU(g) = g (1 - e^-g + ...) -> g
    big = np.full_like(x, 40.0)
    _close(o.rms_swiglu(x, big, w, f32(1e-6)), plain * 40.0, 1e-15, what="saturated gate")
    # the gate does not touch the reduction: rows keep the norm's scale
    one = np.ones_like(x)
    _close(o.rms_swiglu(x, one, w, f32(1e-6)), plain / (1 + np.exp(-1.0)), 1e-14,
           what="unit gate")


PINS = [pin_golden_hand_cases, pin_exact_bruteforce_rms, pin_exact_bruteforce_layer,
        pin_rms_unit_invariant, pin_layer_moments, pin_library_identities,
        pin_special_cases, pin_invariances, pin_affine_structure, pin_row_independence,
        pin_bf16_decoding, pin_f16_decoding, pin_dual, pin_rope_norm_and_identity, pin_rope_relative_position,
        pin_rope_composition_and_scale, pin_rope_layouts_and_table, pin_dual_rope,
        pin_rms_swiglu_bruteforce, pin_rms_swiglu_gate_identities]
