"""Every kernel the dispatch can reach, in both launch forms, once against the
oracle.

For each operation and element type the widths 1-1024, every 16-byte-pack
multiple up to 65536 and a few wider rows are walked through every variant,
aligned and not; each distinct kernel runs at the first width and alignment
that selects it, on a ragged number of rows that spans several blocks of
rows.  The call-level description (the library's own validation and choice
for these tensors) confirms that the kernel under test is the one launched.
The fused RoPE kernels get the same treatment over head sizes 2-4096 (full,
half and two-feature rotations, both pairings)."""
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
OPS = {"rms": trn.OP_RMS, "layer": trn.OP_LAYER, "layer_nobias": trn.OP_LAYER_NOBIAS,
       "dual": trn.OP_DUAL, "gate": trn.OP_RMS_SWIGLU}
DTYPES = {torch.float32: (trn.F32, 4), torch.bfloat16: (trn.BF16, 8),
          torch.float16: (trn.F16, 8)}
BUDGET = 1 << 21        # elements per tensor, at most


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def o():
    return oracle.default()


def kernels(op, code, vec):
    """Distinct kernels (name without the launch form) -> the first (width,
    aligned, variant) that selects each."""
    widths = list(range(1, 1025)) + list(range(1032, 65537, 8)) + [65544, 70000, 1 << 20]
    found = {}
    for w in widths:
        for aligned in (True, False):
            if aligned and w % vec:
                continue
            try:
                n = trn.variant_count(op, code, w, aligned=aligned)
            except trn.FnormError:
                continue
            for v in range(n):
                name = trn.describe(op, code, w, aligned=aligned, variant=v)
                found.setdefault(name.rsplit(".", 1)[0], (w, aligned, v, n))
    return found


def field(name, key):
    for part in name.split("."):
        if part.startswith(key) and part[len(key):].isdigit():
            return int(part[len(key):])
    return None


def rows_for(name, width):
    """Two blocks of rows and a ragged tail, within the element budget."""
    lpr, blk = field(name, "lpr"), field(name, "blk")
    rpb = 1 if ".wide." in name or not lpr else max(1, blk // lpr)
    return max(2, min(2 * rpb + 3, BUDGET // width))


def placed(t, aligned):
    """t on the device; one element past a 16-byte boundary when not aligned."""
    if aligned:
        return t.to(DEV)
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
    view = buf[1:].view(t.shape)
    view.copy_(t.to(DEV))
    return view


def empty_like_placed(t, aligned):
    if aligned:
        return torch.empty(t.shape, dtype=t.dtype, device=DEV)
    return torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)[1:].view(t.shape)


def run_one(o, oname, dtype, width, aligned, variant, expect, seed):
    rows = rows_for(expect, width)
    if oname == "dual":
        # [tokens, heads, head_dim], queries and keys sharing the tokens
        tokens = max(1, rows // 4)
        g = torch.Generator().manual_seed(seed)
        q = (torch.randn(tokens, 3, width, generator=g)).to(dtype)
        k = (torch.randn(tokens, 1, width, generator=g)).to(dtype)
        qw = (1 + 0.1 * torch.randn(width, generator=g)).to(dtype)
        kw = (1 + 0.1 * torch.randn(width, generator=g)).to(dtype)
        dq, dk, dqw, dkw = (placed(t, aligned) for t in (q, k, qw, kw))
        qy, ky = empty_like_placed(q, aligned), empty_like_placed(k, aligned)
        got = trn.describe_dual_call(dq, dk, dqw, dkw, q_out=qy, k_out=ky, variant=variant)
        assert got == expect, (got, expect)
        trn.dual_head_rms_norm(dq, dk, dqw, dkw, 1e-6, q_out=qy, k_out=ky, variant=variant)
        torch.cuda.synchronize()
        rq, rk = o.dual_head_rms(*(helpers.to_oracle_array(t) for t in (q, k, qw, kw)), 1e-6)
        helpers.check("rms", qy.cpu(), rq, label=f"{expect} w={width} q")
        helpers.check("rms", ky.cpu(), rk, label=f"{expect} w={width} k")
        return
    base = {"rms": "rms", "layer": "layer", "layer_nobias": "layer", "gate": "swiglu"}[oname]
    t = inputs.random_rows(base, rows, width, dtype, seed=seed, mean=0.5, std=1.5,
                           with_bias=(oname == "layer"))
    x, w = placed(t["x"], aligned), placed(t["w"], aligned)
    b = placed(t["b"], aligned) if "b" in t else None
    g = placed(t["g"], aligned) if "g" in t else None
    y = empty_like_placed(t["x"], aligned)
    opc = trn.OP_RMS_SWIGLU if oname == "gate" else (trn.OP_RMS if oname == "rms" else trn.OP_LAYER)
    got = trn.describe_call(opc, x, w, b, out=y, g=g, variant=variant)
    assert got == expect, (got, expect)
    eps = 1e-5
    if oname == "gate":
        trn.rms_norm_swiglu(x, g, w, eps, out=y, variant=variant)
    elif oname == "rms":
        trn.rms_norm(x, w, eps, out=y, variant=variant)
    else:
        trn.layer_norm(x, w, b, eps, out=y, variant=variant)
    torch.cuda.synchronize()
    xa, wa = helpers.to_oracle_array(t["x"]), helpers.to_oracle_array(t["w"])
    if oname == "gate":
        r = o.rms_swiglu(xa, helpers.to_oracle_array(t["g"]), wa, eps)
        helpers.check("rms", y.cpu(), r, label=f"{expect} w={width}",
                      floor=np.full(r.shape, 1e-30))
    elif oname == "rms":
        helpers.check_row("rms", y.cpu(), o.rms(xa, wa, eps), label=f"{expect} w={width}")
    else:
        ba = helpers.to_oracle_array(t["b"]) if "b" in t else None
        helpers.check_row("layer", y.cpu(), o.layer(xa, wa, ba, eps), t["w"], t.get("b"),
                          label=f"{expect} w={width}", kernel=expect)


@pytest.mark.parametrize("dtype", list(DTYPES), ids=["f32", "bf16", "f16"])
@pytest.mark.parametrize("oname", list(OPS))
def test_every_kernel(o, oname, dtype):
    code, vec = DTYPES[dtype]
    found = kernels(OPS[oname], code, vec)
    assert found
    say(f"[every] {oname} {dtype}: {len(found)} kernels")
    for i, (kern, (width, aligned, v, n)) in enumerate(sorted(found.items(),
                                                              key=lambda kv: kv[1][0])):
        for var in sorted({v, v ^ 1}):
            if var >= n:
                continue
            expect = trn.describe(OPS[oname], code, width, aligned=aligned, variant=var)
            say(f"[every] {expect} width={width} aligned={aligned} variant={var}")
            run_one(o, oname, dtype, width, aligned, var, expect, seed=7 * i + var)


def rope_kernels(code):
    """Distinct fused RoPE kernels -> the first (head_dim, rotated dims,
    interleaved, aligned, variant, count) that selects each."""
    found = {}
    for hd in range(2, 4097, 2):
        for dims in sorted({hd, hd // 2 if (hd // 2) % 2 == 0 else hd, 2}):
            for trad in (False, True):
                for aligned in (True, False):
                    try:
                        n = trn.rope_variant_count(code, hd, dims, trad, aligned=aligned)
                    except trn.FnormError:
                        continue
                    for v in range(n):
                        name = trn.describe_rope(code, hd, dims, trad, aligned=aligned, variant=v)
                        found.setdefault(name.rsplit(".", 1)[0], (hd, dims, trad, aligned, v, n))
    return found


@pytest.mark.parametrize("dtype", list(DTYPES), ids=["f32", "bf16", "f16"])
def test_every_rope_kernel(o, dtype):
    """Every fused RoPE kernel the dispatch can reach (head sizes 2-4096,
    full, half and two-feature rotations, both pairings, aligned or not), in
    both launch forms, against the oracle: 3 query + 1 key heads per token
    at positions from 1000 on."""
    code, _ = DTYPES[dtype]
    found = rope_kernels(code)
    assert found
    say(f"[every-rope] {dtype}: {len(found)} kernels")
    for i, (kern, (hd, dims, trad, aligned, v, n)) in enumerate(sorted(found.items(),
                                                                     key=lambda kv: kv[1][0])):
        for var in sorted({v, v ^ 1}):
            if var >= n:
                continue
            expect = trn.describe_rope(code, hd, dims, trad, aligned=aligned, variant=var)
            say(f"[every-rope] {expect} head_dim={hd} dims={dims} aligned={aligned} variant={var}")
            rows = rows_for(expect, hd)
            tokens = max(1, rows // 4)
            g = torch.Generator().manual_seed(11 * i + var)
            q = torch.randn(tokens, 3, hd, generator=g).to(dtype)
            k = torch.randn(tokens, 1, hd, generator=g).to(dtype)
            qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype)
            kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype)
            dq, dk, dqw, dkw = (placed(t, aligned) for t in (q, k, qw, kw))
            qy, ky = empty_like_placed(q, aligned), empty_like_placed(k, aligned)
            offset = 1000 + i
            rope = {"dims": dims, "traditional": trad, "offset": offset}
            got = trn.describe_dual_call(dq, dk, dqw, dkw, q_out=qy, k_out=ky, variant=var,
                                         rope=rope)
            assert got == expect, (got, expect)
            trn.dual_head_rms_rope(dq, dk, dqw, dkw, 1e-6, dims=dims, traditional=trad,
                                   offset=offset, q_out=qy, k_out=ky, variant=var)
            torch.cuda.synchronize()
            rq, rk = o.dual_head_rms_rope(*(helpers.to_oracle_array(t) for t in (q, k, qw, kw)),
                                          1e-6, dims, trad, 10000.0, 1.0, offset)
            helpers.check_rope(o, q, k, qw, kw, qy.cpu(), ky.cpu(), rq, rk, dims, trad,
                               f"{expect} hd={hd}", (offset + tokens) / (2 * np.pi))
