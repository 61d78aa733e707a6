"""GPU parity of RMSNorm with the SiLU-gate epilogue (fnorm_rms_swiglu)
against the fp64 oracle, at every element type, across widths (exact,
masked, scalar and wide kernels), every kernel variant, strided and
in-place calls, and the full gated-output-norm workload.

Tolerance: the RMSNorm tolerance of the element type on each output,
relative to max(|r|, 1e-30) (fp16: its usual 2^-14 floor); values whose
gate drives SiLU under fp32's normal range are compared only through that
floor.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_row_normalization_amd as trn
from tests import helpers
from transformer_row_normalization_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = [torch.float32, torch.bfloat16, torch.float16]


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def o():
    return oracle.default()


def bits(t):
    return t.detach().cpu().contiguous().view(torch.uint8)


def ref(o, x, g, w, eps):
    return o.rms_swiglu(*(helpers.to_oracle_array(t.cpu().contiguous()) for t in (x, g, w)), eps)


def check(y, r, label):
    helpers.check("rms", y.cpu(), r, label=label, floor=np.full(r.shape, 1e-30))


def case(rows, width, dtype, seed, extremes=True):
    t = inputs.random_rows("swiglu", rows, width, dtype, seed)
    if extremes:   # saturated gates both ways, and exact zeros
        g = t["g"].float()
        g.view(-1)[::13] = 60.0
        g.view(-1)[5::17] = -60.0
        g.view(-1)[7::19] = 0.0
        t["g"] = g.to(dtype)
    return t


# up to rows past every type's register capacity (fp32 40000, all types at
# 65537 and 70000), which take the strided wide kernel
WIDTHS = [1, 3, 8, 64, 100, 128, 192, 256, 576, 640, 768, 1024, 2560, 4096, 5120, 8192,
          20000, 40000, 65537, 70000]


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: str(d)[6:])
@pytest.mark.parametrize("width", WIDTHS)
def test_matches_oracle(o, width, dtype):
    rows = 37 if width <= 8192 else 5
    say(f"[swiglu] width={width} {dtype} {trn.describe(trn.OP_RMS_SWIGLU, {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[dtype], width)}")
    t = case(rows, width, dtype, seed=width)
    x, g, w = (t[k].to(DEV) for k in ("x", "g", "w"))
    y = trn.rms_norm_swiglu(x, g, w, 1e-6)
    torch.cuda.synchronize()
    check(y, ref(o, t["x"], t["g"], t["w"], 1e-6), f"swiglu {width} {dtype}")


@pytest.mark.parametrize("dtype,width", [(torch.bfloat16, 128), (torch.bfloat16, 4096),
                                         (torch.bfloat16, 8192), (torch.float32, 768),
                                         (torch.float16, 64), (torch.bfloat16, 100)])
def test_every_variant(o, dtype, width):
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[dtype]
    t = case(70, width, dtype, seed=3 * width)
    x, g, w = (t[k].to(DEV) for k in ("x", "g", "w"))
    r = ref(o, t["x"], t["g"], t["w"], 1e-5)
    n = trn.variant_count(trn.OP_RMS_SWIGLU, code, width)
    assert n >= 2
    for v in range(n):
        say(f"[swiglu] {width} {dtype} v{v} {trn.describe(trn.OP_RMS_SWIGLU, code, width, variant=v)}")
        y = trn.rms_norm_swiglu(x, g, w, 1e-5, variant=v)
        torch.cuda.synchronize()
        check(y, r, f"swiglu {width} v{v}")


def test_gate_multiplies_the_plain_norm(o):
    """fp32: the gated output is the plain RMSNorm output times SiLU(g), to a
    few ulp (the same reduction; only the epilogue differs)."""
    t = case(64, 4096, torch.float32, seed=9, extremes=False)
    x, g, w = (t[k].to(DEV) for k in ("x", "g", "w"))
    plain = trn.rms_norm(x, w, 1e-6).double().cpu().numpy()
    gated = trn.rms_norm_swiglu(x, g, w, 1e-6).double().cpu().numpy()
    gd = t["g"].double().numpy()
    expect = plain * gd / (1 + np.exp(-gd))
    err = np.abs(gated - expect) / np.maximum(np.abs(expect), 1e-30)
    assert err.max() < 5e-7, err.max()


def test_strided_and_in_place(o):
    """x and the gate as the two halves of one projection output (row
    stride 2 * width), written back in place over x; then over the gate."""
    for dtype in DTYPES:
        rows, width = 50, 256
        t = case(rows, width, dtype, seed=21)
        proj = torch.empty(rows, 2 * width, dtype=dtype, device=DEV)
        proj[:, :width] = t["x"].to(DEV)
        proj[:, width:] = t["g"].to(DEV)
        w = t["w"].to(DEV)
        r = ref(o, t["x"], t["g"], t["w"], 1e-6)
        x, g = proj[:, :width], proj[:, width:]
        out = trn.rms_norm_swiglu(x, g, w, 1e-6)          # strided in, contiguous out
        torch.cuda.synchronize()
        check(out, r, f"strided {dtype}")
        trn.rms_norm_swiglu(x, g, w, 1e-6, out=x)          # in place over x
        torch.cuda.synchronize()
        assert torch.equal(bits(x), bits(out))
        assert torch.equal(bits(proj[:, width:]), bits(t["g"].to(DEV)))   # gate untouched
        proj[:, :width] = t["x"].to(DEV)
        trn.rms_norm_swiglu(x, g, w, 1e-6, out=g)          # in place over the gate
        torch.cuda.synchronize()
        assert torch.equal(bits(g), bits(out))


def test_deterministic_and_zero_rows(o):
    t = case(300, 1024, torch.bfloat16, seed=4)
    x, g, w = (t[k].to(DEV) for k in ("x", "g", "w"))
    a = trn.rms_norm_swiglu(x, g, w, 1e-5)
    b = trn.rms_norm_swiglu(x, g, w, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))
    e = trn.rms_norm_swiglu(x[:0], g[:0], w, 1e-5)
    assert e.shape == (0, 1024)


def test_full_workload(o):
    """The gated output norm at the dual layout (4096 tokens x 32 heads x
    128), every row against the oracle in chunks."""
    wl = inputs.rms_swiglu_bf16_4096tok()
    t = wl.tensors
    x, g, w = (t[k].to(DEV) for k in ("x", "g", "w"))
    y = trn.rms_norm_swiglu(x, g, w, wl.eps)
    torch.cuda.synchronize()
    y = y.cpu().reshape(-1, 128)
    xs, gs = t["x"].reshape(-1, 128), t["g"].reshape(-1, 128)
    for r0 in range(0, xs.shape[0], 16384):
        r = ref(o, xs[r0:r0 + 16384], gs[r0:r0 + 16384], t["w"], wl.eps)
        check(y[r0:r0 + 16384], r, f"full rows {r0}+")
