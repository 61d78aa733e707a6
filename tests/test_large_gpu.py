"""Tensors past 2^31 elements (64-bit row offsets): RMSNorm and LayerNorm
over 262400 x 8192 bf16 (2.15e9 elements, 4.3 GB in and out), and the dual
head norm over 16.9 million head vectors; rows at the start, at the end and
around element 2^31 are checked against the oracle one by one."""
import sys

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
    helpers.check(op, ys, r, w.cpu(), f"large {op}")
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
