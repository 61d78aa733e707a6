"""The library called from plain C on the GPU (tests/c_abi/gpu_call, built
by build()): every fused entry point, run from C on seeded bf16 inputs, is
bitwise equal to the same call through the Python binding."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import transformer_row_normalization_amd as trn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "gpu_call")


def test_c_program_matches_binding(tmp_path):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build()")
    rows, width, tokens, qh, kh, hd = 96, 4096, 33, 8, 2, 128
    g = torch.Generator().manual_seed(17)
    bf = torch.bfloat16
    t = {"x": torch.randn(rows, width, generator=g).to(bf),
         "g": (2 * torch.randn(rows, width, generator=g)).to(bf),
         "w": (1 + 0.1 * torch.randn(width, generator=g)).to(bf),
         "b": (0.02 * torch.randn(width, generator=g)).to(bf),
         "q": torch.randn(tokens, qh, hd, generator=g).to(bf),
         "k": torch.randn(tokens, kh, hd, generator=g).to(bf),
         "qw": (1 + 0.1 * torch.randn(hd, generator=g)).to(bf),
         "kw": (1 + 0.1 * torch.randn(hd, generator=g)).to(bf)}
    for name, v in t.items():
        v.view(torch.int16).numpy().tofile(tmp_path / f"{name}.bin")
    print(f"[c] gpu_call {rows}x{width}, {tokens} tokens", file=sys.stderr, flush=True)
    out = subprocess.run([EXE, str(tmp_path), str(rows), str(width), str(tokens), str(qh),
                          str(kh), str(hd)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    d = {k: v.to(DEV) for k, v in t.items()}
    want = {"rms": trn.rms_norm(d["x"], d["w"], 1e-5),
            "layer": trn.layer_norm(d["x"], d["w"], d["b"], 1e-5),
            "swiglu": trn.rms_norm_swiglu(d["x"], d["g"], d["w"], 1e-5)}
    want["qy"], want["ky"] = trn.dual_head_rms_norm(d["q"], d["k"], d["qw"], d["kw"], 1e-6)
    want["qr"], want["kr"] = trn.dual_head_rms_rope(d["q"], d["k"], d["qw"], d["kw"], 1e-6,
                                                    offset=5)
    torch.cuda.synchronize()
    for name, ref in want.items():
        got = torch.from_numpy(np.fromfile(tmp_path / f"{name}.bin", dtype=np.int16))
        assert torch.equal(got, ref.cpu().view(torch.int16).reshape(-1)), name
