"""fnorm_rms_composed_noalloc (the composed RMSNorm with its intermediates in
the library's static device scratch) against fnorm_rms_composed (the same
chain with a caller's workspace): bitwise-equal outputs on two calls in a
row, the second smaller, each also checked against the fp64 oracle."""
import pytest
import torch

import oracle
import transformer_row_normalization_amd as trn
from tests import helpers
from transformer_row_normalization_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_noalloc_matches_workspace_form_twice():
    o = oracle.default()
    cases = [("rms", 2048, 2048, torch.bfloat16, 1e-5, 71),   # 4M elements (16 MiB of fp32)
             ("rms", 37, 1000, torch.float32, 1e-6, 72)]      # then a smaller, ragged one
    for _, rows, width, dtype, eps, seed in cases:
        t = inputs.random_rows("rms", rows, width, dtype, seed=seed, mean=0.5, std=1.5)
        x, w = t["x"].to(DEV), t["w"].to(DEV)
        ref = trn.rms_norm_composed(x, w, eps)
        y = trn.rms_norm_composed_noalloc(x, w, eps)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), ref.view(torch.uint8)), (rows, width, dtype)
        r = o.rms(helpers.to_oracle_array(t["x"]), helpers.to_oracle_array(t["w"]), eps)
        helpers.check("rms", y.cpu(), r, label=f"noalloc {rows}x{width}")


def test_noalloc_rejects_beyond_scratch():
    x = torch.empty(4096, 4096, dtype=torch.float32, device=DEV)
    w = torch.empty(4096, dtype=torch.float32, device=DEV)
    with pytest.raises(trn.FnormError, match="WORKSPACE"):
        trn.rms_norm_composed_noalloc(x, w, 1e-6)
