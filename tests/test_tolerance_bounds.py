"""The tolerance machinery of tests/helpers.py, pinned on the CPU.

An fp32 evaluation of LayerNorm written out op by op in numpy float32
(row sums over 16-element lanes and a pairwise tree, as the kernels form
them; the corrected two-pass; fma emulated by one rounding of the exact fp64
value) must pass the LayerNorm bound at the depth of its sums;
a rotation evaluated with sine/cosine errors of the hardware's measured size
must pass the RoPE bound.  Planted mistakes that the former floor (1-ulp
checks only where |r| >= |w_j|) let through must fail: a centring error of
2^-13 of the row's standard deviation, a few outputs off by 3 ulps where the
output cancels, and a rotation by the neighbouring position."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import helpers

F = np.float32


def fl(v):
    """Round fp64 values to fp32 (one rounding)."""
    return np.asarray(v, dtype=np.float64).astype(F)


PER_LANE = 16


def tree_sum(v, square=False):
    """Row sums of v [rows, n] in fp32 the way the kernels form them: each of
    ceil(n / 16) lanes adds its 16 elements one after another (fma for the
    squares), then the lanes are added pairwise.  Returns (sums, depth)."""
    rows, n = v.shape
    lanes = -(-n // PER_LANE)
    lanes2 = 1 << (lanes - 1).bit_length()
    pad = np.zeros((rows, lanes2 * PER_LANE), F)
    pad[:, :n] = v
    pad = pad.reshape(rows, lanes2, PER_LANE)
    acc = np.zeros((rows, lanes2), F)
    for k in range(PER_LANE):
        col = pad[:, :, k]
        acc = fl(col.astype(np.float64) ** 2 + acc) if square else acc + col
    while acc.shape[1] > 1:
        acc = acc[:, 0::2] + acc[:, 1::2]
    return acc[:, 0], PER_LANE + (lanes2.bit_length() - 1)


def layer_f32(x, w, b, eps, centre_error=0.0):
    """LayerNorm of the rows of x in fp32, every operation rounded: the row
    sums as tree_sum forms them, mean, the deviations, their sum and sum of
    squares, c = sum(d)/N, var, 1/sqrt(var + eps), ((x - mean) - c) s, then
    fma with w and b.  Returns (y, depth of the sums)."""
    rows, n = x.shape
    inv = F(1.0 / n)
    acc, depth = tree_sum(x)
    mean = acc * inv
    d = x - mean[:, None]
    sd, _ = tree_sum(d)
    sq, _ = tree_sum(d, square=True)
    c = sd * inv
    var = np.maximum((sq - c * sd) * inv, F(0))
    s = fl(1.0 / np.sqrt((var + F(eps)).astype(np.float64)))
    dd = d - c[:, None]
    if centre_error:
        dd = fl(dd - centre_error * np.sqrt(var.astype(np.float64))[:, None])
    p = dd * s[:, None]
    return fl(p.astype(np.float64) * w + b), depth


def make_rows(seed, rows, width, mean, outliers):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, width, generator=g) + mean
    if outliers:
        x = torch.where(torch.rand(rows, width, generator=g) < 0.01, x * 100, x)
    w = 1 + 0.1 * torch.randn(width, generator=g)
    b = 0.02 * torch.randn(width, generator=g)
    return (x.to(torch.bfloat16), w.to(torch.bfloat16), b.to(torch.bfloat16))


CASES = [(0, 64, 512, 3.0, True), (1, 64, 768, 0.0, False), (2, 32, 1024, 30.0, False)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"w{c[2]}-mean{c[3]}-out{int(c[4])}")
def test_fp32_layernorm_passes_and_mistakes_fail(case):
    seed, rows, width, mean, outliers = case
    x, w, b = make_rows(seed, rows, width, mean, outliers)
    eps = 1e-5
    r = oracle.default().layer(*(helpers.to_oracle_array(t) for t in (x, w, b)), eps)
    x32, w32, b32 = (helpers.widen(t).astype(F) for t in (x, w, b))
    y32, depth = layer_f32(x32, w32, b32, eps)
    # fp32 output: within max(E, 1e-5 |r|)
    e = helpers.check("layer", torch.from_numpy(y32), r, w, "emulated f32", b=b, depth=depth)
    assert e["max_bound_use"] <= 1.0
    # the row's own centring scale (mean|x - mean| s) against its upper bound 1
    e1 = helpers.check("layer", torch.from_numpy(y32), r, w, "emulated f32", b=b, depth=depth,
                       kappa=1.0)
    assert e1["n_checked"] <= e["n_checked"]
    # bf16 output: <= 1 ulp under the bound's rule, which covers nearly every output
    ybf = torch.from_numpy(y32).to(torch.bfloat16)
    e = helpers.check("layer", ybf, r, w, "emulated bf16", b=b, depth=depth)
    assert e["frac_checked"] > 0.99, e
    # a centring error of 2^-13 sd: within the old floor (2^-7 |w_j|), not this bound
    bad, _ = layer_f32(x32, w32, b32, eps, centre_error=2.0 ** -13)
    with pytest.raises(AssertionError):
        helpers.check("layer", torch.from_numpy(bad).to(torch.bfloat16), r, w, "centring", b=b,
                      depth=depth)
    # three outputs off by 3 ulps where |r| < |w_j| (unchecked by the old floor)
    bits = helpers.bf16_bits(ybf).reshape(r.shape).astype(np.int32)
    absr = np.abs(r)
    cand = np.argwhere((absr < np.abs(helpers.widen(w))) & (absr > 0.05))[:3]
    for i, j in cand:
        bits[i, j] += 3 if bits[i, j] < 0x8000 else -3
    planted = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16)
    with pytest.raises(AssertionError):
        helpers.check("layer", planted, r, w, "planted ulps", b=b, depth=depth)


def rotate(plain, pos, dims, base, cos_err, sin_err):
    """Split-half rotation of fp64 head vectors [tokens, heads, hd] at positions
    pos, with absolute errors added to the cosine and sine."""
    half = dims // 2
    i = np.arange(half)
    theta = pos[:, None] * base ** (-2.0 * i / dims)
    c = (np.cos(theta) + cos_err)[:, None, :]
    s = (np.sin(theta) + sin_err)[:, None, :]
    a, p = plain[..., :half], plain[..., half:dims]
    out = plain.copy()
    out[..., :half] = a * c - p * s
    out[..., half:dims] = p * c + a * s
    return out


def test_rope_bound_holds_for_hardware_sized_trig_errors():
    g = torch.Generator().manual_seed(9)
    tokens, qh, kh, hd, offset = 64, 4, 2, 128, 5000
    q = torch.randn(tokens, qh, hd, generator=g).to(torch.bfloat16)
    k = torch.randn(tokens, kh, hd, generator=g).to(torch.bfloat16)
    qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(torch.bfloat16)
    kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(torch.bfloat16)
    o = oracle.default()
    arrs = [helpers.to_oracle_array(t) for t in (q, k, qw, kw)]
    rq, _ = o.dual_head_rms_rope(*arrs, 1e-6, hd, False, 10000.0, 1.0, offset)
    pq, _ = o.dual_head_rms(*arrs, 1e-6)
    pos = offset + np.arange(tokens, dtype=np.float64)
    # normalized values with fp32-sized relative error, worst-case trig errors
    noisy = pq * (1 + 4 * helpers.U32)
    err = helpers.HW_TRIG_ABS_ERR + helpers.TRIG_ARG_ERR
    y = rotate(noisy, pos, hd, 10000.0, err, -err)
    turns = (offset + tokens) / (2 * math.pi)
    bound = helpers.rope_bound(rq, pq, hd, False, 22, turns)
    for dt in (torch.float32, torch.bfloat16):
        yt = torch.from_numpy(y.astype(np.float32)).to(dt)
        e = helpers.check("rms", yt, rq, label=f"rope {dt}", bound=bound)
        if dt == torch.bfloat16:
            assert e["frac_checked"] > 0.99, e
    # the neighbouring position's rotation fails
    shifted = rotate(pq, pos + 1, hd, 10000.0, 0.0, 0.0)
    with pytest.raises(AssertionError):
        helpers.check("rms", torch.from_numpy(shifted.astype(np.float32)).to(torch.bfloat16), rq,
                      label="shifted", bound=bound)


def test_kernel_depth_parses_names():
    assert helpers.kernel_depth("layer.bf16.vec8.vpt4.lpr128.blk256.exact.nt.persistent2", 4096) \
        == 32 + 6 + 1
    assert helpers.kernel_depth("dual.bf16.vec8.vpt2.lpr8.blk256.exact.nt.grid", 128) == 16 + 3
    assert helpers.kernel_depth("rms.f32.vec4.wide.blk1024.persistent", 40000) == 40 + 6 + 15
    assert helpers.kernel_depth("layer.bf16.vec1.vpt4.lpr1024.blk1024.masked.persistent", 4096) \
        == 4 + 6 + 15



def test_fp16_subnormal_outputs_under_the_bound_check():
    """Below fp16's smallest normal (2^-14) the spacing is a fixed 2^-24, so
    under 2^-15 even the correctly rounded value can be more than 2^-10 off
    relatively (half a step of 2^-24 against |r| < 512 steps).  The bound
    check takes relative error against 2^-14 there: the correctly rounded
    value and its neighbour toward r pass (ulp distance 0 and 1), a value two
    steps away fails."""
    step = 2.0 ** -24
    r = np.array([486.49 * step, -(300.45 * step), 1.5 + 0.49 * 2.0 ** -10])
    bound = np.full(r.shape, 1e-12)               # the fp32 value is all but exact
    rne = r.astype(np.float16).astype(np.float64)
    spacing = np.where(np.abs(r) < 2.0 ** -14, step, 2.0 ** -10)   # 1.5 is in [1, 2)
    toward = np.sign(r - rne)
    for y, ulps in ((rne, 0), (rne + toward * spacing, 1)):
        out = helpers.check("rms", torch.tensor(y, dtype=torch.float16), r, label=f"{ulps} ulp",
                            bound=bound)
        assert out["max_ulp"] == ulps and out["max_rel"] <= helpers.F16_REL_TOL
    with pytest.raises(AssertionError):
        helpers.check("rms", torch.tensor(rne + 2 * toward * spacing, dtype=torch.float16), r,
                      label="two steps", bound=bound)
