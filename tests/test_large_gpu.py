"""Tensors past 2^31 elements (64-bit row offsets): RMSNorm and LayerNorm
over 262400 x 8192 bf16 (2.15e9 elements, 4.3 GB in and out), and the dual
head norm over 16.9 million head vectors; rows at the start, at the end and
around element 2^31 are checked against the oracle one by one.  And past
2^31 rows (head vectors), where the kernels divide a row index by the head
count in 64 bits: the fused RoPE and the dual on a packed QKV buffer."""
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


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def o():
    return oracle.default()


def sample_rows(rows, width):
    edge = (1 << 31) // width
    idx = list(range(0, 48)) + list(range(edge - 24, edge + 24)) + list(range(rows - 48, rows))
    return torch.tensor(sorted(set(i for i in idx if 0 <= i < rows)))


@pytest.mark.parametrize("op", ["rms", "layer"])
def test_rows_past_2_31_elements(o, op):
    rows, width = 262400, 8192
    assert rows * width > (1 << 31)
    say(f"[large] {op} {rows}x{width} bf16 ({rows * width} elements)")
    t = inputs.large_rows_on_device(rows, width, torch.bfloat16, seed=31, device=DEV,
                                    mean=1.0 if op == "layer" else 0.0)
    x, w, b = t["x"], t["w"], t["b"]
    y = trn.rms_norm(x, w, 1e-5) if op == "rms" else trn.layer_norm(x, w, b, 1e-5)
    torch.cuda.synchronize()
    idx = sample_rows(rows, width).to(DEV)
    xs, ys = x.index_select(0, idx).cpu(), y.index_select(0, idx).cpu()
    wa = helpers.to_oracle_array(w.cpu())
    if op == "rms":
        r = o.rms(helpers.to_oracle_array(xs), wa, 1e-5)
    else:
        r = o.layer(helpers.to_oracle_array(xs), wa, helpers.to_oracle_array(b.cpu()), 1e-5)
    helpers.check_row(op, ys, r, w.cpu(), None if op == "rms" else b.cpu(), f"large {op}")
    del x, y, t
    torch.cuda.empty_cache()


def test_dual_past_2_31_elements(o):
    tokens, qh, kh, hd = 420000, 32, 8, 128
    assert tokens * (qh + kh) * hd > (1 << 31)
    say(f"[large] dual {tokens} tokens x ({qh}+{kh}) heads x {hd}")
    tq = inputs.large_rows_on_device(tokens * qh, hd, torch.bfloat16, seed=32, device=DEV)
    tk = inputs.large_rows_on_device(tokens * kh, hd, torch.bfloat16, seed=33, device=DEV)
    q, k = tq["x"].view(tokens, qh, hd), tk["x"].view(tokens, kh, hd)
    qw, kw = tq["w"], tk["w"]
    qy, ky = trn.dual_head_rms_norm(q, k, qw, kw, 1e-6)
    torch.cuda.synchronize()
    for name, src, out, wt, n in (("q", tq["x"], qy, qw, tokens * qh), ("k", tk["x"], ky, kw, tokens * kh)):
        idx = sample_rows(n, hd).to(DEV)
        r = o.rms(helpers.to_oracle_array(src.index_select(0, idx).cpu()),
                  helpers.to_oracle_array(wt.cpu()), 1e-6)
        helpers.check("rms", out.view(-1, hd).index_select(0, idx).cpu(), r, label=f"large dual {name}")
    del q, k, qy, ky, tq, tk
    torch.cuda.empty_cache()


def test_rope_past_2_31_rows(o):
    """More than 2^31 head vectors in one tensor: the fused RoPE kernel then
    divides a row index by the head count in 64 bits (the multiply-high
    division covers rows below 2^31 only).  32 query + 8 key heads of 4
    features (the scalar-access kernel), positions offset by 1000; tokens at
    the start, around query row 2^31 and at the end against the oracle."""
    tokens, qh, kh, hd, offset = (1 << 26) + 2, 32, 8, 4, 1000
    assert tokens * qh > (1 << 31)
    say(f"[large] rope {tokens} tokens x ({qh}+{kh}) heads x {hd}")
    tq = inputs.large_rows_on_device(tokens * qh, hd, torch.bfloat16, seed=34, device=DEV)
    tk = inputs.large_rows_on_device(tokens * kh, hd, torch.bfloat16, seed=35, device=DEV)
    q, k = tq["x"].view(tokens, qh, hd), tk["x"].view(tokens, kh, hd)
    qw, kw = tq["w"], tk["w"]
    yq, yk = trn.dual_head_rms_rope(q, k, qw, kw, 1e-6, offset=offset)
    torch.cuda.synchronize()
    edge = (1 << 31) // qh                      # the token holding query row 2^31
    toks = sorted(set([0, 1, 2] + list(range(edge - 3, edge + 2)) + [tokens - 2, tokens - 1]))
    idx = torch.tensor(toks, device=DEV)
    qs, ks = q.index_select(0, idx).cpu(), k.index_select(0, idx).cpu()
    yqs, yks = yq.index_select(0, idx).cpu(), yk.index_select(0, idx).cpu()
    qwc, kwc = qw.cpu(), kw.cpu()
    rq, rk = [], []
    for i, t in enumerate(toks):                # each sampled token at its own position
        a, b = o.dual_head_rms_rope(helpers.to_oracle_array(qs[i:i + 1]),
                                    helpers.to_oracle_array(ks[i:i + 1]),
                                    helpers.to_oracle_array(qwc), helpers.to_oracle_array(kwc),
                                    1e-6, hd, False, 10000.0, 1.0, offset + t)
        rq.append(a)
        rk.append(b)
    helpers.check_rope(o, qs, ks, qwc, kwc, yqs, yks, np.concatenate(rq), np.concatenate(rk),
                       hd, False, "large rope", (offset + tokens) / (2 * np.pi))
    del q, k, yq, yk, tq, tk
    torch.cuda.empty_cache()


def test_packed_dual_past_2_31_rows(o):
    """The dual head norm on the q and k parts of one packed [tokens, q + 2k
    heads, head_dim] buffer with more than 2^31 query rows: each row's token
    comes from a 64-bit division by the head count."""
    tokens, qh, kh, hd = (1 << 26) + 2, 32, 8, 4
    heads = qh + 2 * kh
    assert tokens * qh > (1 << 31)
    say(f"[large] packed dual {tokens} tokens x {heads} heads x {hd}")
    t = inputs.large_rows_on_device(tokens * heads, hd, torch.bfloat16, seed=36, device=DEV)
    buf = t["x"].view(tokens, heads, hd)
    q, k = buf[:, :qh], buf[:, qh:qh + kh]
    w2 = inputs.large_rows_on_device(1, hd, torch.bfloat16, seed=37, device=DEV)["w"]
    qw, kw = t["w"], w2
    qy, ky = trn.dual_head_rms_norm(q, k, qw, kw, 1e-6)
    torch.cuda.synchronize()
    edge = (1 << 31) // qh
    toks = sorted(set([0, 1] + list(range(edge - 2, edge + 2)) + [tokens - 1]))
    idx = torch.tensor(toks, device=DEV)
    for name, src, out, wt in (("q", q, qy, qw), ("k", k, ky, kw)):
        xs = src.index_select(0, idx).reshape(-1, hd).cpu()
        r = o.rms(helpers.to_oracle_array(xs), helpers.to_oracle_array(wt.cpu()), 1e-6)
        helpers.check("rms", out.index_select(0, idx).reshape(-1, hd).cpu(), r,
                      label=f"large packed dual {name}")
    del buf, q, k, qy, ky, t
    torch.cuda.empty_cache()
