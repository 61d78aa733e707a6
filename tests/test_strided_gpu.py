"""GPU parity of the row-strided entry points: rows that are views into a
wider buffer, and the query/key parts of one packed QKV buffer normalized in
place (with and without the fused RoPE).

Each strided result is checked against the fp64 oracle on the same rows
(made contiguous on the host), and bitwise against the contiguous entry
point, which runs the same kernel; the bytes between rows must be left as
they were.
"""
import re
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


def oracle_rows(o, op, x, w, b, eps):
    xa, wa = helpers.to_oracle_array(x.cpu()), helpers.to_oracle_array(w.cpu())
    if op == "rms":
        return o.rms(xa, wa, eps)
    return o.layer(xa, wa, None if b is None else helpers.to_oracle_array(b.cpu()), eps)


def run(op, x, w, b, eps, out=None, variant=-1):
    if op == "rms":
        return trn.rms_norm(x, w, eps, out=out, variant=variant)
    return trn.layer_norm(x, w, b, eps, out=out, variant=variant)


DCODE = {torch.float32: trn.F32, torch.bfloat16: trn.BF16, torch.float16: trn.F16}

STRIDE_CASES = [  # (op, width, x row stride, x column offset, y row stride, y column offset)
    ("rms", 128, 384, 128, 256, 64),        # heads of a packed buffer
    ("rms", 4096, 4096 + 64, 32, 4096, 0),  # padded rows into a packed output
    ("layer", 768, 2304, 768, 1024, 8),
    ("layer", 1000, 1003, 1, 1000, 0),      # odd stride: scalar-access kernels
    ("rms", 8192, 8192 + 8, 0, 8192 + 8, 0),
    ("rms", 100, 128, 0, 120, 4),
    ("layer", 33, 40, 3, 35, 1),
    ("rms", 20000, 20480, 0, 20000, 0),     # beyond one workgroup's registers
]


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: str(d)[6:])
@pytest.mark.parametrize("case", STRIDE_CASES, ids=lambda c: f"{c[0]}-w{c[1]}-s{c[2]}/{c[4]}")
def test_row_strided_matches_oracle_and_contiguous(o, case, dtype):
    op, width, xs, xc, ys, yc = case
    rows = 77
    eb = torch.finfo(dtype).bits // 8
    say(f"[strided] {op} {dtype} width={width} x stride {xs}+{xc} y stride {ys}+{yc}")
    t = inputs.random_rows(op, rows, width, dtype, seed=width + xs)
    w = t["w"].to(DEV)
    b = t["b"].to(DEV) if op == "layer" else None
    xbuf = torch.full((rows, xs), float("nan"), dtype=dtype, device=DEV)
    x = xbuf[:, xc:xc + width]
    x.copy_(t["x"].to(DEV))
    ybuf = torch.full((rows, ys), 7.0, dtype=dtype, device=DEV)
    y = ybuf[:, yc:yc + width]
    opc = trn.OP_RMS if op == "rms" else trn.OP_LAYER
    name = trn.describe_call(opc, x, w, b, out=y)
    got = run(op, x, w, b, 1e-5, out=y)
    assert got.data_ptr() == y.data_ptr()
    ref = run(op, t["x"].to(DEV), w, b, 1e-5)
    torch.cuda.synchronize()
    helpers.check_row(op, y.cpu(), oracle_rows(o, op, t["x"], t["w"], t.get("b"), 1e-5),
                      t["w"], t.get("b"), f"strided {op} {width}")
    aligned = (xs * eb) % 16 == 0 and (ys * eb) % 16 == 0 and (xc * eb) % 16 == 0 \
        and (yc * eb) % 16 == 0
    # the library names the kernel this strided call took: the contiguous
    # call's when every pointer and stride is 16-byte aligned, else the
    # scalar-access kernel
    contiguous = trn.describe_call(opc, t["x"].to(DEV), w, b)
    if aligned:   # the same kernel as the contiguous call
        assert name == contiguous, (name, contiguous)
        assert torch.equal(bits(y), bits(ref))
    else:
        assert ".vec1." in name and name == trn.describe(opc, DCODE[dtype], width, aligned=False)
    # the bytes around the rows are untouched
    mask = torch.ones(rows, ys, dtype=torch.bool)
    mask[:, yc:yc + width] = False
    assert torch.all(ybuf.cpu()[mask] == 7.0)
    assert torch.all(torch.isnan(xbuf.cpu()[mask_x(rows, xs, xc, width)]))


def mask_x(rows, xs, xc, width):
    m = torch.ones(rows, xs, dtype=torch.bool)
    m[:, xc:xc + width] = False
    return m


@pytest.mark.parametrize("op", ["rms", "layer"])
def test_row_strided_every_variant(o, op):
    """Every kernel variant serving the width, on strided rows."""
    dtype, width, rows, xs = torch.bfloat16, 1024, 300, 1536
    code = trn.BF16
    t = inputs.random_rows(op, rows, width, dtype, seed=11)
    w = t["w"].to(DEV)
    b = t["b"].to(DEV) if op == "layer" else None
    xbuf = torch.zeros(rows, xs, dtype=dtype, device=DEV)
    x = xbuf[:, 256:256 + width]
    x.copy_(t["x"].to(DEV))
    r = oracle_rows(o, op, t["x"], t["w"], t.get("b"), 1e-5)
    n = trn.variant_count(trn.OP_RMS if op == "rms" else trn.OP_LAYER, code, width)
    for v in range(n):
        say(f"[strided] {op} variant {v}: {trn.describe(trn.OP_RMS if op == 'rms' else trn.OP_LAYER, code, width, variant=v)}")
        ybuf = torch.zeros(rows, xs, dtype=dtype, device=DEV)
        y = ybuf[:, 512:512 + width]
        run(op, x, w, b, 1e-5, out=y, variant=v)
        torch.cuda.synchronize()
        helpers.check_row(op, y.cpu(), r, t["w"], t.get("b"), f"strided {op} v{v}")
        assert torch.all(ybuf[:, :512].cpu() == 0) and torch.all(ybuf[:, 512 + width:].cpu() == 0)


def test_row_strided_in_place(o):
    """In place on every other row of a buffer: the other rows keep their values."""
    for dtype in DTYPES:
        t = inputs.random_rows("rms", 64, 2048, dtype, seed=3)
        buf = t["x"].to(DEV).clone()
        x = buf[::2]
        before_odd = buf[1::2].clone()
        trn.rms_norm(x, t["w"].to(DEV), 1e-6, out=x)
        torch.cuda.synchronize()
        helpers.check("rms", x.cpu(), oracle_rows(o, "rms", t["x"][::2], t["w"], None, 1e-6),
                      label=f"in place strided {dtype}")
        assert torch.equal(bits(buf[1::2]), bits(before_odd))




def fresh(t):
    """A contiguous copy that never shares t's storage (a view that is
    already contiguous would come back as itself from .contiguous())."""
    return t.clone(memory_format=torch.contiguous_format)


def packed_qkv(tokens, qh, kh, hd, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    buf = torch.randn(tokens, (qh + 2 * kh) * hd, generator=g).to(dtype).to(DEV)
    q = buf[:, :qh * hd].view(tokens, qh, hd)
    k = buf[:, qh * hd:(qh + kh) * hd].view(tokens, kh, hd)
    v = buf[:, (qh + kh) * hd:].view(tokens, kh, hd)
    qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype).to(DEV)
    kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype).to(DEV)
    return buf, q, k, v, qw, kw


QKV_CASES = [  # (dtype, tokens, q_heads, k_heads, head_dim)
    (torch.bfloat16, 257, 32, 8, 128),
    (torch.float16, 64, 16, 4, 64),
    (torch.float32, 33, 8, 2, 256),
    (torch.bfloat16, 1, 32, 8, 128),
    (torch.bfloat16, 19, 6, 2, 100),       # head_dim that masks
    (torch.bfloat16, 41, 7, 3, 128),       # head counts that are not powers of two
    (torch.float32, 23, 40, 5, 64),
]


@pytest.mark.parametrize("case", QKV_CASES, ids=lambda c: f"{str(c[0])[6:]}-t{c[1]}-h{c[2]}/{c[3]}-hd{c[4]}")
def test_packed_qkv_dual_in_place(o, case):
    dtype, tokens, qh, kh, hd = case
    say(f"[qkv dual] {case}")
    buf, q, k, v, qw, kw = packed_qkv(tokens, qh, kh, hd, dtype, seed=tokens + hd)
    q0, k0, v0 = fresh(q), fresh(k), fresh(v)
    ref_q, ref_k = trn.dual_head_rms_norm(q0, k0, qw, kw, 1e-6)
    # packed views whose token stride is a 16-byte multiple take the
    # contiguous call's kernel
    name = trn.describe_dual_call(q, k, qw, kw, q_out=q, k_out=k)
    eb = torch.finfo(dtype).bits // 8
    if (q.stride(0) * eb) % 16 == 0 and (qh * hd * eb) % 16 == 0 and (hd * eb) % 16 == 0:
        assert name == trn.describe_dual_call(q0, k0, qw, kw), name
    else:
        assert ".vec1." in name, name
    yq, yk = trn.dual_head_rms_norm(q, k, qw, kw, 1e-6, q_out=q, k_out=k)
    torch.cuda.synchronize()
    assert yq.data_ptr() == q.data_ptr() and yk.data_ptr() == k.data_ptr()
    rq, rk = o.dual_head_rms(*(helpers.to_oracle_array(t.cpu()) for t in (q0, k0, qw, kw)), 1e-6)
    helpers.check("rms", q.cpu(), rq, label="packed q")
    helpers.check("rms", k.cpu(), rk, label="packed k")
    assert torch.equal(bits(q), bits(ref_q)) and torch.equal(bits(k), bits(ref_k))
    assert torch.equal(bits(v), bits(v0))


@pytest.mark.parametrize("case", QKV_CASES, ids=lambda c: f"{str(c[0])[6:]}-t{c[1]}-h{c[2]}/{c[3]}-hd{c[4]}")
def test_packed_qkv_rope_in_place(o, case):
    dtype, tokens, qh, kh, hd = case
    for trad in (False, True):
        say(f"[qkv rope] {case} traditional={trad}")
        buf, q, k, v, qw, kw = packed_qkv(tokens, qh, kh, hd, dtype, seed=tokens + hd + trad)
        q0, k0, v0 = fresh(q), fresh(k), fresh(v)
        kwargs = dict(dims=hd, traditional=trad, base=10000.0, scale=1.0, offset=37)
        if trn.rope_variant_count(DCODE[dtype], hd, hd, trad) == 0:
            # a head shape the fused kernel does not serve: refused, not run
            with pytest.raises(trn.FnormError, match="UNSUPPORTED"):
                trn.dual_head_rms_rope(q, k, qw, kw, 1e-6, q_out=q, k_out=k, **kwargs)
            assert torch.equal(bits(q), bits(q0)) and torch.equal(bits(k), bits(k0))
            continue
        ref_q, ref_k = trn.dual_head_rms_rope(q0, k0, qw, kw, 1e-6, **kwargs)
        trn.dual_head_rms_rope(q, k, qw, kw, 1e-6, q_out=q, k_out=k, **kwargs)
        torch.cuda.synchronize()
        rq, rk = o.dual_head_rms_rope(*(helpers.to_oracle_array(t.cpu()) for t in (q0, k0, qw, kw)),
                                      1e-6, hd, trad, 10000.0, 1.0, 37)
        helpers.check_rope(o, q0.cpu(), k0.cpu(), qw.cpu(), kw.cpu(), q.cpu(), k.cpu(), rq, rk,
                           hd, trad, "packed rope", (37 + tokens) / (2 * np.pi))
        assert torch.equal(bits(q), bits(ref_q)) and torch.equal(bits(k), bits(ref_k))
        assert torch.equal(bits(v), bits(v0))


def test_packed_qkv_to_separate_outputs(o):
    """Strided inputs, contiguous outputs; and contiguous inputs written
    into a packed output buffer."""
    dtype, tokens, qh, kh, hd = torch.bfloat16, 100, 8, 2, 128
    buf, q, k, v, qw, kw = packed_qkv(tokens, qh, kh, hd, dtype, seed=1)
    ref_q, ref_k = trn.dual_head_rms_norm(fresh(q), fresh(k), qw, kw, 1e-6)
    yq, yk = trn.dual_head_rms_norm(q, k, qw, kw, 1e-6)
    assert yq.is_contiguous() and yk.is_contiguous()
    out = torch.zeros_like(buf)
    oq = out[:, :qh * hd].view(tokens, qh, hd)
    ok = out[:, qh * hd:(qh + kh) * hd].view(tokens, kh, hd)
    trn.dual_head_rms_norm(fresh(q), fresh(k), qw, kw, 1e-6, q_out=oq, k_out=ok)
    torch.cuda.synchronize()
    for a, b_ in ((yq, ref_q), (yk, ref_k), (oq, ref_q), (ok, ref_k)):
        assert torch.equal(bits(a), bits(b_))
    assert torch.all(out[:, (qh + kh) * hd:].cpu() == 0)


def _variant_named(opc, code, width, aligned, name):
    for v in range(trn.variant_count(opc, code, width, aligned)):
        if trn.describe(opc, code, width, aligned, v) == name:
            return v
    raise AssertionError(f"no variant named {name}")


@pytest.mark.parametrize("case", ["aligned", "misaligned", "odd_stride", "in_place", "no_bias"])
def test_describe_call_names_the_kernel_that_runs(case):
    """describe_call's answer is the kernel the call launches: forcing the
    variant of that name gives bitwise the default call's output, and the
    widths here are served by shapes with different reduction trees."""
    dtype, rows, width = torch.bfloat16, 96, 4096
    code = trn.BF16
    t = inputs.random_rows("layer", rows, width, dtype, seed=17, mean=1.0, std=2.0)
    w, b = t["w"].to(DEV), t["b"].to(DEV)
    if case == "misaligned":
        xbuf = torch.empty(rows * width + 1, dtype=dtype, device=DEV)
        x = xbuf[1:].view(rows, width)
        x.copy_(t["x"].to(DEV))
    elif case == "odd_stride":
        xbuf = torch.empty(rows, width + 3, dtype=dtype, device=DEV)
        x = xbuf[:, :width]
        x.copy_(t["x"].to(DEV))
    else:
        x = t["x"].to(DEV).clone()
    if case == "no_bias":
        b = None
    aligned = case not in ("misaligned", "odd_stride")
    opc = trn.OP_LAYER if b is not None else trn.OP_LAYER_NOBIAS
    out = x if case == "in_place" else torch.empty(rows, width, dtype=dtype, device=DEV)
    name = trn.describe_call(trn.OP_LAYER, x, w, b, out=out)
    assert (".vec1." in name) == (not aligned), name
    v = _variant_named(opc, code, width, aligned, name)
    say(f"[describe] {case}: {name} (variant {v})")
    x0 = x.clone()
    y_default = trn.layer_norm(x, w, b, 1e-5, out=out).clone()
    if case == "in_place":
        x.copy_(x0)
    y_forced = trn.layer_norm(x, w, b, 1e-5, out=out, variant=v)
    torch.cuda.synchronize()
    assert torch.equal(bits(y_default), bits(y_forced))
    if not aligned:
        # the scalar-access shapes for this width (one element per access, 4
        # per thread, 1024 lanes; and the wide kernel, 1024 threads striding by
        # 1024) add the same elements in the same order: nothing to tell apart
        return
    # a kernel with another reduction tree (packs per lane, lanes per row)
    # for the same width computes in a different order
    def tree(n):
        return tuple(re.findall(r"(?<=\.)(vec\d+|vpt\d+|lpr\d+|wide)(?=\.)", n))
    other = next(u for u in range(trn.variant_count(opc, code, width, aligned))
                 if tree(trn.describe(opc, code, width, aligned, u)) != tree(name))
    if case == "in_place":
        x.copy_(x0)
    y_other = trn.layer_norm(x, w, b, 1e-5, out=out, variant=other)
    torch.cuda.synchronize()
    assert not torch.equal(bits(y_default), bits(y_other)), "shapes not distinguishable here"
