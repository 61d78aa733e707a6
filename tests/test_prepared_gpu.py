"""Prepared calls (validate once, relaunch through the C entry point):
every launch gives the bitwise result of the plain call on the current
contents of the bound tensors; invalid arguments fail at preparation."""
import pytest
import torch

import transformer_row_normalization_amd as trn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t):
    return t.detach().cpu().contiguous().view(torch.uint8)


def test_prepared_ops_match_plain_calls():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(64, 4096, generator=g).to(torch.bfloat16).to(DEV)
    gate = torch.randn(64, 4096, generator=g).to(torch.bfloat16).to(DEV)
    w = (1 + 0.1 * torch.randn(4096, generator=g)).to(torch.bfloat16).to(DEV)
    b = (0.02 * torch.randn(4096, generator=g)).to(torch.bfloat16).to(DEV)
    q = torch.randn(4, 32, 128, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(4, 8, 128, generator=g).to(torch.bfloat16).to(DEV)
    qw = (1 + 0.1 * torch.randn(128, generator=g)).to(torch.bfloat16).to(DEV)
    kw = (1 + 0.1 * torch.randn(128, generator=g)).to(torch.bfloat16).to(DEV)
    cases = [
        (trn.rms_norm, (x, w, 1e-5), {}),
        (trn.layer_norm, (x, w, b, 1e-5), {}),
        (trn.rms_norm_swiglu, (x, gate, w, 1e-5), {}),
        (trn.dual_head_rms_norm, (q, k, qw, kw, 1e-6), {}),
        (trn.dual_head_rms_rope, (q, k, qw, kw, 1e-6), {"offset": 77}),
        (trn.dual_head_rms_norm, (q[:, :8], k, qw, kw, 1e-6), {}),      # strided views
    ]
    for op, args, kw_ in cases:
        launch, out = trn.prepare(op, *args, **kw_)
        outs = out if isinstance(out, tuple) else (out,)
        want = op(*args, **kw_)
        wants = want if isinstance(want, tuple) else (want,)
        torch.cuda.synchronize()
        for o, r in zip(outs, wants):
            assert torch.equal(bits(o), bits(r)), op.__name__
        for o in outs:
            o.zero_()
        launch()
        launch()
        torch.cuda.synchronize()
        for o, r in zip(outs, wants):
            assert torch.equal(bits(o), bits(r)), op.__name__ + " relaunch"


def test_prepared_launch_reads_current_contents():
    x = torch.randn(8, 1024, device=DEV)
    w = torch.ones(1024, device=DEV)
    launch, y = trn.prepare(trn.rms_norm, x, w, 1e-6)
    x.mul_(-3.0)
    launch()
    ref = trn.rms_norm(x, w, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(ref))


def test_prepare_validates_in_the_library():
    x = torch.randn(8, 1024, device=DEV)
    w = torch.ones(1024, device=DEV)
    with pytest.raises(trn.FnormError, match="EPS"):
        trn.prepare(trn.rms_norm, x, w, -1.0)
    # an output overlapping its input without being it: the library refuses
    # it when the prepared call is first launched
    buf = torch.randn(8 * 1024 + 8, device=DEV)
    xin, yout = buf[:8 * 1024].view(8, 1024), buf[8:].view(8, 1024)
    with pytest.raises(trn.FnormError, match="ALIAS"):
        trn.prepare(trn.rms_norm, xin, w, 1e-6, out=yout)
