"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances (tests/helpers.py): RMSNorm fp32 relative error <= 1e-5, bf16
<= 1 ulp from the correctly rounded oracle value and <= 2^-7 relative, at
every output.  LayerNorm and RoPE outputs, which can cancel, against a bound
derived from the fp32 evaluation (<= 1 ulp wherever that bound is below a
half ulp; within the bound elsewhere).  Bitwise checks where the contract is
bitwise: dual == two single calls, null bias == zero bias, run-to-run
determinism.  The full-size workloads report their ulp histograms.
"""
import sys
import threading

import numpy as np
import pytest
import torch

import oracle
import transformer_row_normalization_amd as trn
from tests import helpers
from transformer_row_normalization_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def dcode(dtype):
    return {torch.float32: trn.F32, torch.bfloat16: trn.BF16, torch.float16: trn.F16}[dtype]


@pytest.fixture(scope="module")
def o():
    return oracle.default()


def run_oracle(o, op, t, eps):
    if op == "rms":
        return o.rms(helpers.to_oracle_array(t["x"]), helpers.to_oracle_array(t["w"]), eps)
    b = t.get("b")
    return o.layer(helpers.to_oracle_array(t["x"]), helpers.to_oracle_array(t["w"]),
                   None if b is None else helpers.to_oracle_array(b), eps)


def run_gpu(op, t, eps, variant=-1, out=None):
    x = t["x"].to(DEV)
    w = t["w"].to(DEV)
    if op == "rms":
        y = trn.rms_norm(x, w, eps, out=out, variant=variant)
    else:
        b = t.get("b")
        y = trn.layer_norm(x, w, None if b is None else b.to(DEV), eps, out=out, variant=variant)
    torch.cuda.synchronize()
    return y.cpu()


def check(op, y, r, t, label, kappa=None, kernel=None):
    """helpers.check_row for a row op on the tensors `t` (x, w, optional b)."""
    return helpers.check_row(op, y, r, t["w"], t.get("b"), label, kappa, kernel)


def default_kernel(op, t):
    """Name of the kernel a contiguous, aligned call on `t` launches."""
    x = t["x"]
    opc = trn.OP_RMS if op == "rms" else (trn.OP_LAYER if t.get("b") is not None
                                          else trn.OP_LAYER_NOBIAS)
    return trn.describe(opc, dcode(x.dtype), x.shape[-1])


def compare_chunked(o, op, t, y, eps, label, chunk_rows=1024):
    """Element-by-element comparison of every output row, in row chunks;
    returns the merged error figures and ulp histograms."""
    x, w, b = t["x"], t["w"], t.get("b")
    width = x.shape[-1]
    x2 = x.reshape(-1, width)
    y2 = y.reshape(-1, width)
    acc = None
    kernel = default_kernel(op, t)
    for r0 in range(0, x2.shape[0], chunk_rows):
        part = {"x": x2[r0:r0 + chunk_rows], "w": w}
        if b is not None:
            part["b"] = b
        r = run_oracle(o, op, part, eps)
        e = check(op, y2[r0:r0 + chunk_rows], r, part, f"{label} rows {r0}+", kernel=kernel)
        acc = helpers.merge_stats(acc, e)
    return acc


# ----------------------------------------------------------------- configs
@pytest.mark.parametrize("variant", ["uniform", "iota"])
def test_rms_f32_512x1024(o, variant):
    wl = inputs.rms_f32_512x1024(variant)
    say(f"[parity] {wl.name}")
    y = run_gpu("rms", wl.tensors, wl.eps)
    e = compare_chunked(o, "rms", wl.tensors, y, wl.eps, wl.name)
    helpers.report(f"{wl.name}-{variant}", e)
    # the Emily notebook expects composed-vs-fused differences of order 1e-5
    assert e["max_abs"] <= 1e-5, e


def test_layer_f32_1024x768(o):
    wl = inputs.layer_f32_1024x768()
    say(f"[parity] {wl.name}")
    y = run_gpu("layer", wl.tensors, wl.eps)
    e = compare_chunked(o, "layer", wl.tensors, y, wl.eps, wl.name)
    helpers.report(wl.name, e)
    # ffai-argus kernel_micro_ab asserts fused-vs-library agreement < 1e-4
    assert e["max_abs"] < 1e-4, e


def test_dual_bf16_4096tok(o):
    wl = inputs.dual_bf16_4096tok()
    t = wl.tensors
    say(f"[parity] {wl.name}")
    q, k, qw, kw = (t[n].to(DEV) for n in ("q", "k", "qw", "kw"))
    qy, ky = trn.dual_head_rms_norm(q, k, qw, kw, wl.eps)
    torch.cuda.synchronize()
    rq, rk = o.dual_head_rms(*(helpers.to_oracle_array(t[n]) for n in ("q", "k", "qw", "kw")),
                             wl.eps)
    helpers.report(f"{wl.name}-queries", helpers.check("rms", qy.cpu(), rq, label="dual queries"))
    helpers.report(f"{wl.name}-keys", helpers.check("rms", ky.cpu(), rk, label="dual keys"))
    # one launch gives bitwise the results of two single launches
    sq = trn.rms_norm(q, qw, wl.eps)
    sk = trn.rms_norm(k, kw, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(qy.view(torch.int16), sq.view(torch.int16))
    assert torch.equal(ky.view(torch.int16), sk.view(torch.int16))


def test_rms_bf16_16384x8192(o):
    wl = inputs.rms_bf16_16384x8192()
    say(f"[parity] {wl.name}")
    y = run_gpu("rms", wl.tensors, wl.eps)
    helpers.report(wl.name, compare_chunked(o, "rms", wl.tensors, y, wl.eps, wl.name))


def test_layer_bf16_65536x4096(o):
    wl = inputs.layer_bf16_65536x4096()
    say(f"[parity] {wl.name} outliers={wl.tensors['outliers']}")
    t = {k: v for k, v in wl.tensors.items() if k in ("x", "w", "b")}
    y = run_gpu("layer", t, wl.eps)
    helpers.report(wl.name, compare_chunked(o, "layer", t, y, wl.eps, wl.name, chunk_rows=2048))


# ----------------------------------------------------------------- sweeps
SWEEP_WIDTHS = [1, 2, 3, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255,
                256, 257, 384, 511, 512, 513, 640, 767, 768, 769, 1000, 1023, 1024, 1536, 2047,
                2048, 2056, 3000, 4095, 4096, 4104, 5120, 8191, 8192, 8200, 12288, 16384,
                18432, 24576, 32768]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16],
                         ids=["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["rms", "layer", "layer_nobias"])
def test_width_sweep(o, op, dtype):
    for i, width in enumerate(SWEEP_WIDTHS):
        rows = 37 if width <= 4096 else 9      # ragged: not a multiple of rows per block
        base = "layer" if op.startswith("layer") else "rms"
        t = inputs.random_rows(base, rows, width, dtype, seed=1000 + i, mean=0.5, std=1.5,
                               with_bias=(op == "layer"))
        eps = 1e-5
        say(f"[sweep] {op} {dtype} rows={rows} width={width} "
            f"kernel={trn.describe(trn.OP_RMS if base == 'rms' else trn.OP_LAYER, dcode(dtype), width)}")
        y = run_gpu(base, t, eps)
        check(base, y, run_oracle(o, base, t, eps), t, f"{op} w={width}")


VARIANT_CASES = [("rms", torch.bfloat16, 128), ("rms", torch.bfloat16, 768),
                 ("rms", torch.bfloat16, 1024), ("rms", torch.bfloat16, 4096),
                 ("rms", torch.bfloat16, 8192), ("rms", torch.float32, 768),
                 ("rms", torch.float32, 1024), ("rms", torch.float32, 4096),
                 ("layer", torch.bfloat16, 4096), ("layer", torch.bfloat16, 8192),
                 ("layer", torch.float32, 768), ("layer", torch.float32, 1024),
                 ("layer", torch.bfloat16, 2048), ("rms", torch.float32, 8192),
                 ("layer", torch.bfloat16, 100), ("rms", torch.float32, 3),
                 ("rms", torch.float16, 4096), ("layer", torch.float16, 4096),
                 ("rms", torch.float16, 8192), ("layer", torch.float16, 768),
                 ("layer", torch.bfloat16, 5120), ("rms", torch.bfloat16, 2560),
                 ("layer", torch.float32, 4096), ("rms", torch.float16, 16384),
                 ("layer", torch.bfloat16, 3584), ("layer", torch.bfloat16, 18432),
                 ("rms", torch.float32, 12288), ("layer", torch.bfloat16, 40960),
                 ("layer", torch.float32, 24576), ("layer", torch.bfloat16, 360),
                 ("rms", torch.float32, 180), ("layer", torch.bfloat16, 6144),
                 ("layer", torch.float32, 3000), ("layer", torch.bfloat16, 24576),
                 ("layer", torch.bfloat16, 192), ("rms", torch.float32, 96),
                 ("layer", torch.bfloat16, 576), ("layer", torch.float32, 320),
                 ("rms", torch.bfloat16, 576), ("rms", torch.bfloat16, 640),
                 ("rms", torch.float32, 288), ("rms", torch.bfloat16, 192),
                 ("layer", torch.bfloat16, 256), ("layer", torch.float32, 128),
                 ("rms", torch.float16, 256)]


@pytest.mark.parametrize("op,dtype,width", VARIANT_CASES,
                         ids=[f"{a}-{str(b)[6:]}-{c}" for a, b, c in VARIANT_CASES])
def test_every_variant(o, op, dtype, width):
    """Every kernel the dispatch table offers for the shape, both grid policies."""
    rows = 301
    t = inputs.random_rows(op, rows, width, dtype, seed=width, mean=1.0, std=2.0)
    eps = 1e-5
    r = run_oracle(o, op, t, eps)
    code = dcode(dtype)
    opc = trn.OP_RMS if op == "rms" else trn.OP_LAYER
    n = trn.variant_count(opc, code, width)
    assert n >= 4
    for v in range(n):
        name = trn.describe(opc, code, width, variant=v)
        say(f"[variant] {op} {dtype} width={width} v={v} {name}")
        y = run_gpu(op, t, eps, variant=v)
        check(op, y, r, t, f"{op} w={width} variant {v}", kernel=name)


# head sizes of models, odd ones, and the large dual shapes (rows over one,
# two, four and sixteen wavefronts with a cross-wave LDS reduction, up to the
# largest head each type serves: 65536 for 2-byte types, 32768 for fp32)
@pytest.mark.parametrize("hd", [64, 80, 96, 128, 192, 256, 100, 512, 576, 640, 1024, 2048,
                                4096, 8192, 16384, 32768, 65536])
def test_dual_equals_two_singles(o, hd):
    tokens = 33 if hd <= 1024 else 3
    for dtype in (torch.bfloat16, torch.float32, torch.float16):
        code = dcode(dtype)
        n = trn.variant_count(trn.OP_DUAL, code, hd)
        if dtype == torch.float32 and hd > 32768:
            assert n == 0          # past fp32's largest dual head: refused
            continue
        g = torch.Generator().manual_seed(hd)
        q = torch.randn(tokens, 5, hd, generator=g).to(dtype).to(DEV)
        k = torch.randn(tokens, 2, hd, generator=g).to(dtype).to(DEV)
        qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype).to(DEV)
        kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype).to(DEV)
        say(f"[dual] hd={hd} {dtype} variants={n}")
        sq = trn.rms_norm(q, qw, 1e-6)
        sk = trn.rms_norm(k, kw, 1e-6)
        rq, rk = o.dual_head_rms(*(helpers.to_oracle_array(t.cpu()) for t in (q, k, qw, kw)),
                                 1e-6)
        for v in range(n):
            qy, ky = trn.dual_head_rms_norm(q, k, qw, kw, 1e-6, variant=v)
            torch.cuda.synchronize()
            helpers.check("rms", qy.cpu(), rq, label=f"dual q hd={hd} v={v}")
            helpers.check("rms", ky.cpu(), rk, label=f"dual k hd={hd} v={v}")
            if v < 2:   # the default kernel shape is the one fnorm_rms uses
                assert torch.equal(qy.cpu().view(torch.uint8), sq.cpu().view(torch.uint8))
                assert torch.equal(ky.cpu().view(torch.uint8), sk.cpu().view(torch.uint8))


def test_dual_one_side_empty(o):
    g = torch.Generator().manual_seed(5)
    q = torch.randn(16, 4, 128, generator=g).to(torch.bfloat16).to(DEV)
    qw = torch.randn(128, generator=g).to(torch.bfloat16).to(DEV)
    k0 = torch.empty(0, 2, 128, dtype=torch.bfloat16, device=DEV)
    qy, ky = trn.dual_head_rms_norm(q, k0, qw, qw, 1e-6)
    torch.cuda.synchronize()
    assert ky.numel() == 0
    assert torch.equal(qy.view(torch.int16), trn.rms_norm(q, qw, 1e-6).view(torch.int16))
    qy2, ky2 = trn.dual_head_rms_norm(k0, q, qw, qw, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(ky2.view(torch.int16), qy.view(torch.int16))


# ----------------------------------------------------------------- edge cases
def test_rows_zero_one_two(o):
    for rows in (0, 1, 2):
        for op in ("rms", "layer"):
            t = inputs.random_rows(op, rows, 4096, torch.bfloat16, seed=rows)
            y = run_gpu(op, t, 1e-5)
            assert y.shape == (rows, 4096)
            if rows:
                check(op, y, run_oracle(o, op, t, 1e-5), t, f"{op} rows={rows}")


def test_misaligned_pointers(o):
    """Tensors that start one element past a 16-byte boundary use the
    scalar-access kernels and give the same results."""
    for dtype in (torch.float32, torch.bfloat16, torch.float16):
        for op in ("rms", "layer"):
            t = inputs.random_rows(op, 50, 1024, dtype, seed=77)
            big = torch.empty(50 * 1024 + 1, dtype=dtype, device=DEV)
            x = big[1:].view(50, 1024)
            x.copy_(t["x"].to(DEV))
            wbig = torch.empty(1025, dtype=dtype, device=DEV)
            w = wbig[1:]
            w.copy_(t["w"].to(DEV))
            ybig = torch.empty(50 * 1024 + 1, dtype=dtype, device=DEV)
            y = ybig[1:].view(50, 1024)
            if op == "rms":
                name = trn.describe_call(trn.OP_RMS, x, w, out=y)
                trn.rms_norm(x, w, 1e-5, out=y)
            else:
                bbig = torch.empty(1025, dtype=dtype, device=DEV)
                b = bbig[1:]
                b.copy_(t["b"].to(DEV))
                name = trn.describe_call(trn.OP_LAYER, x, w, b, out=y)
                trn.layer_norm(x, w, b, 1e-5, out=y)
            torch.cuda.synchronize()
            # the library's own answer for this call: the scalar-access kernel
            assert ".vec1." in name, name
            assert name == trn.describe(trn.OP_RMS if op == "rms" else trn.OP_LAYER, dcode(dtype),
                                        1024, aligned=False)
            check(op, y.cpu(), run_oracle(o, op, t, 1e-5), t, f"misaligned {op}")


def test_in_place(o):
    for op in ("rms", "layer"):
        for width in (128, 4096, 8192, 1000, 20000):
            t = inputs.random_rows(op, 20, width, torch.bfloat16, seed=width)
            x = t["x"].to(DEV).clone()
            w, b = t["w"].to(DEV), t.get("b")
            b = None if op == "rms" else b.to(DEV)
            opc = trn.OP_RMS if op == "rms" else trn.OP_LAYER
            # in place takes the kernel of the out-of-place call
            assert trn.describe_call(opc, x, w, b, out=x) == trn.describe_call(
                opc, x, w, b, out=torch.empty_like(x))
            if op == "rms":
                trn.rms_norm(x, w, 1e-5, out=x)
            else:
                trn.layer_norm(x, w, b, 1e-5, out=x)
            torch.cuda.synchronize()
            check(op, x.cpu(), run_oracle(o, op, t, 1e-5), t, f"in place {op} {width}")


def test_null_bias_equals_zero_bias():
    for dtype in (torch.float32, torch.bfloat16):
        for width in (768, 4096, 1000):
            t = inputs.random_rows("layer", 64, width, dtype, seed=3)
            x, w = t["x"].to(DEV), t["w"].to(DEV)
            # include exact-mean entries (x == mean gives signed zeros) with negative weights
            x[:, :4] = 2.0
            x[5] = 2.0
            w[:8] = -w[:8].abs()
            y0 = trn.layer_norm(x, w, None, 1e-5)
            y1 = trn.layer_norm(x, w, torch.zeros_like(w), 1e-5)
            torch.cuda.synchronize()
            assert torch.equal(y0.view(torch.uint8), y1.view(torch.uint8))


def test_deterministic():
    wl = inputs.layer_bf16_65536x4096(rows=4096)
    x, w, b = (wl.tensors[n].to(DEV) for n in ("x", "w", "b"))
    y0 = trn.layer_norm(x, w, b, wl.eps)
    y1 = trn.layer_norm(x, w, b, wl.eps)
    r0 = trn.rms_norm(x, w, wl.eps)
    r1 = trn.rms_norm(x, w, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(r0.view(torch.int16), r1.view(torch.int16))


@pytest.mark.parametrize("op,dtype,width", [("rms", torch.bfloat16, 128), ("layer", torch.bfloat16, 360),
                                             ("layer", torch.bfloat16, 5120), ("rms", torch.bfloat16, 12288),
                                             ("layer", torch.float32, 3000), ("layer", torch.bfloat16, 4096),
                                             ("rms", torch.bfloat16, 18432)])
def test_launch_forms_bitwise_equal(op, dtype, width):
    """The two launch forms of one kernel (variants 2i and 2i + 1: a plain grid,
    with or without a resident limit, and a persistent grid) compute every row
    with the same code, so their outputs are bitwise equal; rows chosen so the
    persistent grid loops several times and the plain grid is far larger than
    what fits at once."""
    rows = max(64, (48 << 20) // (width * torch.tensor([], dtype=dtype).element_size()))
    t = inputs.random_rows(op, rows, width, dtype, seed=width + 1, mean=0.5, std=1.5)
    code = dcode(dtype)
    opc = trn.OP_RMS if op == "rms" else trn.OP_LAYER
    say(f"[forms] {op} {dtype} rows={rows} width={width} {trn.describe(opc, code, width, variant=0)}")
    y0 = run_gpu(op, t, 1e-5, variant=0)
    y1 = run_gpu(op, t, 1e-5, variant=1)
    assert trn.describe(opc, code, width, variant=0).rsplit(".", 1)[0] == \
        trn.describe(opc, code, width, variant=1).rsplit(".", 1)[0]
    assert torch.equal(y0.view(torch.int16 if dtype != torch.float32 else torch.int32),
                       y1.view(torch.int16 if dtype != torch.float32 else torch.int32))


@pytest.mark.parametrize("hd,trad", [(128, False), (128, True), (256, False), (64, False)])
def test_rope_launch_forms_bitwise_equal(hd, trad):
    """The fused RoPE launch's two forms (plain and persistent grid) run the
    same kernel: bitwise-equal outputs over 2048 tokens of 32 + 8 heads."""
    g = torch.Generator(device="cpu").manual_seed(hd + int(trad))
    q = torch.randn(2048, 32, hd, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(2048, 8, hd, generator=g).to(torch.bfloat16).to(DEV)
    qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(torch.bfloat16).to(DEV)
    kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(torch.bfloat16).to(DEV)
    say(f"[rope forms] hd={hd} trad={trad} {trn.describe_rope(trn.BF16, hd, hd, trad, variant=0)}")
    a = trn.dual_head_rms_rope(q, k, qw, kw, 1e-6, traditional=trad, offset=77, variant=0)
    b = trn.dual_head_rms_rope(q, k, qw, kw, 1e-6, traditional=trad, offset=77, variant=1)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_special_rows(o):
    """Zero rows, constant rows, NaN and infinity propagate as the oracle says."""
    for dtype in (torch.float32, torch.bfloat16, torch.float16):
        x = torch.randn(8, 256).to(dtype)
        x[1] = 0.0                    # zero row: RMS gives zeros
        x[2] = 3.0                    # constant row: LayerNorm gives the bias
        x[3, 7] = float("nan")        # NaN poisons its row only
        x[4, 9] = float("inf")
        w = (1 + 0.1 * torch.randn(256)).to(dtype)
        b = (0.02 * torch.randn(256)).to(dtype)
        t = {"x": x, "w": w, "b": b}
        for op in ("rms", "layer"):
            y = run_gpu(op, t, 1e-5)
            check(op, y, run_oracle(o, op, t, 1e-5), t, f"special {op}")
        y = run_gpu("layer", t, 1e-5)
        assert torch.equal(y[2].view(torch.uint8), b.view(torch.uint8))


def test_large_mean_stability(o):
    """LayerNorm rows with a mean far from zero (two-pass variance)."""
    for dtype, mean in ((torch.float32, 1000.0), (torch.bfloat16, 300.0)):
        t = inputs.random_rows("layer", 64, 4096, dtype, seed=11, mean=mean, std=1.0)
        y = run_gpu("layer", t, 1e-5)
        check("layer", y, run_oracle(o, "layer", t, 1e-5), t, f"mean {mean}")


def test_magnitude_range(o):
    """Rows scaled by 1e-15 .. 1e15 (eps > 0 and eps = 0): inside fp32's
    range for the sum of squares at width 4096 (|x| up to ~2.9e17), every
    result matches the oracle."""
    base = inputs.random_rows("layer", 16, 4096, torch.float32, seed=5)
    for dtype in (torch.float32, torch.bfloat16):
        for scale in (1e-15, 1e-5, 1e5, 1e15):
            for eps in (1e-6, 0.0):
                t = {"x": (base["x"] * scale).to(dtype), "w": base["w"].to(dtype),
                     "b": (base["b"] * scale).to(dtype)}
                for op in ("rms", "layer"):
                    y = run_gpu(op, t, eps)
                    check(op, y, run_oracle(o, op, t, eps), t,
                          f"{op} scale {scale:g} eps {eps} {dtype}")


def test_wide_rows(o):
    # widths past the register capacity (strided passes over the row), up to
    # rows of about a million features (fp16 2^20 + 3, a ragged width: the
    # scalar-access kernel, ~1000 steps of 1024 threads per pass)
    for dtype, width in ((torch.float32, 40000), (torch.bfloat16, 70000), (torch.bfloat16, 65537),
                         (torch.float16, (1 << 20) + 3)):
        for op in ("rms", "layer"):
            t = inputs.random_rows(op, 5, width, dtype, seed=width)
            say(f"[wide] {op} {dtype} width={width}")
            y = run_gpu(op, t, 1e-5)
            check(op, y, run_oracle(o, op, t, 1e-5), t, f"wide {op} {width}")


def test_concurrent_streams(o):
    """Two host threads, two streams, no shared state."""
    ts = [inputs.random_rows("rms", 2048, 4096, torch.bfloat16, seed=s) for s in (1, 2)]
    dev = [{k: v.to(DEV) for k, v in t.items()} for t in ts]
    ref = [trn.rms_norm(d["x"], d["w"], 1e-5) for d in dev]
    torch.cuda.synchronize()
    outs = [None, None]

    def work(i):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(20):
                outs[i] = trn.rms_norm(dev[i]["x"], dev[i]["w"], 1e-5)
        s.synchronize()

    th = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    for i in range(2):
        assert torch.equal(outs[i].view(torch.int16), ref[i].view(torch.int16))


def test_bench_copy():
    src = torch.randint(0, 1 << 30, (1 << 20,), dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    trn.bench_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_device_memory():
    d = trn.device_memory()
    assert d["memory_clock_khz"] > 0 and d["memory_bus_bits"] > 0
    assert d["compute_units"] == torch.cuda.get_device_properties(0).multi_processor_count


def test_describe_matches_hot_configs():
    assert ".exact" in trn.describe(trn.OP_RMS, trn.BF16, 8192)
    assert ".exact" in trn.describe(trn.OP_LAYER, trn.BF16, 4096)
    assert ".exact" in trn.describe(trn.OP_DUAL, trn.BF16, 128)


# ----------------------------------------------------------------- composed baselines
COMPOSED_CASES = [("rms", torch.float32, 512, 1024), ("layer", torch.float32, 1024, 768),
                  ("rms", torch.float16, 256, 4096), ("layer", torch.float16, 100, 1000),
                  ("rms", torch.bfloat16, 1024, 8192), ("layer", torch.bfloat16, 2048, 4096),
                  ("rms", torch.bfloat16, 37, 100), ("layer", torch.float32, 37, 1001),
                  ("layer", torch.bfloat16, 64, 128), ("rms", torch.float32, 3, 7)]


@pytest.mark.parametrize("op,dtype,rows,width", COMPOSED_CASES,
                         ids=[f"{a}-{str(b)[6:]}-{c}x{d}" for a, b, c, d in COMPOSED_CASES])
def test_composed_chain_matches_oracle(o, op, dtype, rows, width):
    t = inputs.random_rows(op, rows, width, dtype, seed=rows + width, mean=0.5, std=1.5)
    say(f"[composed] {op} {dtype} {rows}x{width}")
    x, w = t["x"].to(DEV), t["w"].to(DEV)
    if op == "rms":
        y = trn.rms_norm_composed(x, w, 1e-5)
    else:
        y = trn.layer_norm_composed(x, w, t["b"].to(DEV), 1e-5)
    torch.cuda.synchronize()
    # the composed chain's mean is not corrected, so its centring error scales
    # with mean|x| / sqrt(var) per row, and its reductions are its own
    kappa = helpers.composed_kappa(t["x"]) if op == "layer" else 1.0
    d = helpers.composed_depth(width)
    if op == "rms":
        check(op, y.cpu(), run_oracle(o, op, t, 1e-5), t, f"composed {op}")
    else:
        helpers.check("layer", y.cpu(), run_oracle(o, op, t, 1e-5), t["w"], f"composed {op}",
                      b=t["b"], depth=d, kappa=kappa)
        y0 = trn.layer_norm_composed(x, w, None, 1e-5)
        torch.cuda.synchronize()
        t0 = {"x": t["x"], "w": t["w"]}
        helpers.check("layer", y0.cpu(), run_oracle(o, op, t0, 1e-5), t["w"], "composed no bias",
                      depth=d, kappa=kappa)


def test_composed_iota_page_case(o):
    """The notebook's Part 1 correctness input: composed and fused agree
    closely (the page expects differences of order 1e-5)."""
    wl = inputs.rms_f32_512x1024("iota")
    x, w = wl.tensors["x"].to(DEV), wl.tensors["w"].to(DEV)
    yc = trn.rms_norm_composed(x, w, wl.eps)
    yf = trn.rms_norm(x, w, wl.eps)
    torch.cuda.synchronize()
    assert float((yc - yf).abs().max()) <= 1e-5
    helpers.check("rms", yc.cpu(), run_oracle(o, "rms", wl.tensors, wl.eps), label="composed iota")


# ----------------------------------------------------------------- dual norm + RoPE
ROPE_CASES = [  # (dtype, tokens, q_heads, k_heads, head_dim, dims, traditional, base, scale, offset, table)
    (torch.bfloat16, 200, 32, 8, 128, 128, False, 10000.0, 1.0, 0, False),
    (torch.bfloat16, 200, 32, 8, 128, 128, True, 10000.0, 1.0, 4000, False),
    (torch.float32, 97, 4, 2, 128, 128, False, 500000.0, 1.0, 131072, False),
    (torch.float32, 97, 4, 2, 128, 64, True, 10000.0, 0.5, 7, False),
    (torch.bfloat16, 64, 16, 4, 64, 64, False, 10000.0, 1.0, 100, True),
    (torch.bfloat16, 33, 8, 8, 256, 256, False, 1000000.0, 1.0, 3, False),
    (torch.bfloat16, 33, 8, 2, 256, 32, False, 10000.0, 1.0, 3, False),
    (torch.bfloat16, 50, 6, 2, 96, 96, False, 10000.0, 1.0, 11, False),
    (torch.float32, 50, 6, 2, 80, 80, True, 10000.0, 2.0, 11, True),
    (torch.bfloat16, 21, 3, 1, 100, 100, True, 10000.0, 1.0, 5, False),
    (torch.float32, 17, 2, 1, 1024, 1024, False, 10000.0, 1.0, 12345, False),
    (torch.bfloat16, 1, 1, 0, 128, 128, False, 10000.0, 1.0, 9, False),
    (torch.bfloat16, 5, 0, 4, 128, 128, True, 10000.0, 1.0, 9, False),
    (torch.float16, 130, 32, 8, 128, 128, False, 10000.0, 1.0, 2048, False),
    (torch.float16, 40, 4, 4, 64, 64, True, 10000.0, 1.0, 3, False),
    # head counts that are not powers of two (the token index is a division)
    (torch.bfloat16, 37, 7, 5, 128, 128, False, 10000.0, 1.0, 77, False),
    (torch.float32, 19, 40, 10, 64, 64, True, 10000.0, 1.0, 1000, False),
    # long contexts: the angle is formed in fp64 and reduced in turns
    (torch.float32, 24, 4, 2, 128, 128, False, 10000.0, 1.0, 1 << 24, False),
    (torch.bfloat16, 24, 8, 2, 128, 128, True, 1000000.0, 1.0, 1000000, False),
    # more than 256 frequency pairs: the host table's later pairs come from
    # its step factors; and a caller's table of 512 pairs
    (torch.bfloat16, 9, 2, 1, 2048, 2048, False, 10000.0, 1.0, 777, False),
    (torch.float32, 7, 2, 1, 1024, 1024, False, 10000.0, 1.0, 5, True),
    # partial rotation on shapes with several packs per lane (the pairing is
    # then chosen at run time): half the features of head_dim 256 and 512
    (torch.bfloat16, 29, 6, 2, 256, 128, False, 10000.0, 1.0, 31, False),
    (torch.bfloat16, 13, 4, 1, 512, 256, False, 500000.0, 1.0, 8, False),
    # split-half rows wider than 128 features fetch a lane's first two
    # frequencies before the row loop: full rotation past 128 pairs, a
    # caller's table, and partial rotation with a second entry on half the lanes
    (torch.bfloat16, 11, 4, 2, 512, 512, False, 10000.0, 1.0, 65537, False),
    (torch.bfloat16, 21, 4, 2, 256, 256, False, 10000.0, 1.0, 99, True),
    (torch.bfloat16, 15, 5, 3, 256, 192, False, 10000.0, 1.0, 4096, False),
    (torch.float32, 9, 3, 2, 256, 192, False, 10000.0, 1.0, 123, True),
    # head_dim 256 in fp16 (split-half) and interleaved bf16: the 4- and
    # 2-pack shapes run as variants of every case
    (torch.float16, 17, 6, 2, 256, 256, False, 10000.0, 1.0, 321, False),
    (torch.bfloat16, 19, 4, 2, 256, 256, True, 10000.0, 1.0, 55, False),
    # the largest rotation served: 2048 pairs at head_dim 4096 (one row per
    # wavefront, an angle table that fills the 64 KB LDS limit; pairs past
    # 256 take the step factors)
    (torch.bfloat16, 5, 2, 1, 4096, 4096, False, 10000.0, 1.0, 300, False),
    (torch.float16, 3, 2, 1, 4096, 4096, True, 500000.0, 1.0, 7, True),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: f"{str(c[0])[6:]}-t{c[1]}-h{c[2]}/{c[3]}-hd{c[4]}-d{c[5]}-{'il' if c[6] else 'sh'}-o{c[9]}{'-tab' if c[10] else ''}")
def test_dual_rope_matches_oracle(o, case):
    dtype, tokens, qh, kh, hd, dims, trad, base, scale, offset, table = case
    g = torch.Generator().manual_seed(hd * 7 + dims)
    q = torch.randn(tokens, qh, hd, generator=g).to(dtype)
    k = torch.randn(tokens, kh, hd, generator=g).to(dtype)
    qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype)
    kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype)
    freqs = None
    if table:
        freqs = (base ** (-torch.arange(0, dims, 2, dtype=torch.float64) / dims)
                 * (1 + 0.3 * torch.rand(dims // 2, generator=g, dtype=torch.float64))).float()
    code = dcode(dtype)
    n = trn.rope_variant_count(code, hd, dims, trad)
    assert n >= 2
    rq, rk = o.dual_head_rms_rope(helpers.to_oracle_array(q), helpers.to_oracle_array(k),
                                  helpers.to_oracle_array(qw), helpers.to_oracle_array(kw),
                                  1e-6, dims, trad, base, scale, offset,
                                  None if freqs is None else freqs.numpy())
    # largest angle in turns: position * scale * inverse frequency (<= 1) / 2 pi
    max_turns = (offset + tokens) * abs(scale) * (
        1.0 if freqs is None else float(freqs.abs().max())) / (2 * np.pi)
    dq, dk, dqw, dkw = (t.to(DEV) for t in (q, k, qw, kw))
    dfr = None if freqs is None else freqs.to(DEV)
    plain_q, plain_k = trn.dual_head_rms_norm(dq, dk, dqw, dkw, 1e-6)
    for v in range(n):
        say(f"[rope] {case} v={v} {trn.describe_rope(code, hd, dims, trad, variant=v)}")
        yq, yk = trn.dual_head_rms_rope(dq, dk, dqw, dkw, 1e-6, dims=dims, traditional=trad,
                                        base=base, scale=scale, offset=offset, freqs=dfr,
                                        variant=v)
        torch.cuda.synchronize()
        e = helpers.check_rope(o, q, k, qw, kw, yq.cpu(), yk.cpu(), rq, rk, dims, trad,
                               f"rope v{v}", max_turns)
        if v == 0:
            for side, st in e.items():
                helpers.report(f"rope-{case[0]}-t{tokens}-hd{hd}-d{dims}-"
                               f"{'il' if trad else 'sh'}-o{offset}-{side}", st)
        if offset == 0 and tokens > 0:
            # token 0 sits at position 0: bitwise the plain dual norm
            assert torch.equal(yq[0].cpu().view(torch.uint8), plain_q[0].cpu().view(torch.uint8))
            assert torch.equal(yk[0].cpu().view(torch.uint8), plain_k[0].cpu().view(torch.uint8))


def test_dual_rope_full_size(o):
    """The dual workload's full shape with RoPE (positions 0..4095)."""
    wl = inputs.dual_bf16_4096tok()
    t = wl.tensors
    q, k, qw, kw = (t[n].to(DEV) for n in ("q", "k", "qw", "kw"))
    yq, yk = trn.dual_head_rms_rope(q, k, qw, kw, wl.eps)
    torch.cuda.synchronize()
    rq, rk = o.dual_head_rms_rope(*(helpers.to_oracle_array(t[n]) for n in ("q", "k", "qw", "kw")),
                                  wl.eps, 128, False, 10000.0, 1.0, 0)
    e = helpers.check_rope(o, t["q"], t["k"], t["qw"], t["kw"], yq.cpu(), yk.cpu(), rq, rk, 128,
                           False, "rope full", 4096 / (2 * np.pi), wl.eps)
    for side, st in e.items():
        helpers.report(f"{wl.name}-rope-{side}", st)
