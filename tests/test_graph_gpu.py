"""Decode-sized calls captured in a HIP graph: every replay must give the
eager results bit for bit, including after the inputs are overwritten in
place between replays (the graph reads the live buffers).

Shapes: one decode step of the dual workload's head layout (tokens 1, 8
and 64; 32 query heads, 8 key heads, head_dim 128), plus RMSNorm and
LayerNorm rows of a hidden state of 4096.  The library's calls queue kernel
launches only (no memset, no allocation), so they can be captured.
"""
import sys

import pytest
import torch

import transformer_row_normalization_amd as trn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def bits(t):
    return t.detach().cpu().contiguous().view(torch.uint8)


@pytest.mark.parametrize("tokens", [1, 8, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32],
                         ids=lambda d: str(d)[6:])
def test_graph_replays_match_eager(tokens, dtype):
    say(f"[graph] tokens={tokens} {dtype}")
    g = torch.Generator().manual_seed(tokens)
    qh, kh, hd, hidden = 32, 8, 128, 4096
    q = torch.randn(tokens, qh, hd, generator=g).to(dtype).to(DEV)
    k = torch.randn(tokens, kh, hd, generator=g).to(dtype).to(DEV)
    qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype).to(DEV)
    kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(dtype).to(DEV)
    h = torch.randn(tokens, hidden, generator=g).to(dtype).to(DEV)
    hw = (1 + 0.1 * torch.randn(hidden, generator=g)).to(dtype).to(DEV)
    hb = (0.02 * torch.randn(hidden, generator=g)).to(dtype).to(DEV)
    outs = {n: torch.empty_like(t) for n, t in
            (("qy", q), ("ky", k), ("qr", q), ("kr", k), ("hr", h), ("hl", h))}

    def step():
        trn.dual_head_rms_norm(q, k, qw, kw, 1e-6, q_out=outs["qy"], k_out=outs["ky"])
        trn.dual_head_rms_rope(q, k, qw, kw, 1e-6, offset=1000, q_out=outs["qr"],
                               k_out=outs["kr"])
        trn.rms_norm(h, hw, 1e-5, out=outs["hr"])
        trn.layer_norm(h, hw, hb, 1e-5, out=outs["hl"])

    def eager():
        step()
        torch.cuda.synchronize()
        return {n: bits(t) for n, t in outs.items()}

    want = eager()
    graph = torch.cuda.CUDAGraph()
    step()                                   # warm the side stream's first use
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(bits(t), want[n]), f"replay {rep}: {n} differs"
    # new inputs written in place: the replay follows them
    q.mul_(-2.0)
    k.add_(0.5)
    h.mul_(3.0)
    want2 = eager()
    for t in outs.values():
        t.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for n, t in outs.items():
        assert torch.equal(bits(t), want2[n]), f"replay after new inputs: {n} differs"
    assert not torch.equal(want2["qy"], want["qy"])
