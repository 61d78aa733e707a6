"""Writes hand_cases.json: exact values of the hand cases, computed only with
the exact-rational oracle (oracle/exact_tiny.py).

Inputs come from the pages:
  - Emily.Fast API docs, `rms_norm` example: x = [[1, 2, 3, 4]], weight ones,
    eps 1e-5 (the docs assert only the output shape; the values are the
    definition evaluated exactly).
  - Emily.Fast API docs, `layer_norm` example: the same x, weight ones, bias
    zeros, eps 1e-5.
  - Emily notebook, Part 1 correctness cell: x = iota/100, weight ones,
    eps 1e-6; here its first two rows at width 8 (the cell's own width, 1024,
    is covered by the fp64 oracle tests).
Plus a few cases with non-trivial weight and bias so that the affine step is
pinned too.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import exact_tiny  # noqa: E402


def f32(v):
    return float(np.float32(v))


def main():
    cases = []
    x = [1.0, 2.0, 3.0, 4.0]
    cases.append({"name": "rms_doc_example", "op": "rms",
                  "source": "Emily.Fast docs, rms_norm, Examples",
                  "x": [x], "w": [1.0] * 4, "eps_f32": f32(1e-5),
                  "y": exact_tiny.rms([x], [1.0] * 4, f32(1e-5))})
    cases.append({"name": "layer_doc_example", "op": "layer",
                  "source": "Emily.Fast docs, layer_norm, Examples",
                  "x": [x], "w": [1.0] * 4, "b": [0.0] * 4, "eps_f32": f32(1e-5),
                  "y": exact_tiny.layer([x], [1.0] * 4, [0.0] * 4, f32(1e-5))})
    iota = [[f32(f32(i) / f32(100.0)) for i in range(r * 8, r * 8 + 8)] for r in range(2)]
    cases.append({"name": "rms_iota_over_100_w8", "op": "rms",
                  "source": "Emily notebook, Part 1, Correctness (iota / 100, ones, eps 1e-6)",
                  "x": iota, "w": [1.0] * 8, "eps_f32": f32(1e-6),
                  "y": exact_tiny.rms(iota, [1.0] * 8, f32(1e-6))})
    xw = [[0.5, -1.25, 2.0, 0.75, -3.0], [10.0, 10.5, 9.5, 10.25, 9.75]]
    w = [1.5, 0.5, -2.0, 1.0, 0.25]
    b = [0.125, -0.5, 0.0, 1.0, -0.0625]
    cases.append({"name": "rms_weighted", "op": "rms",
                  "source": "Emily.Fast docs, rms_norm (weight broadcast over rows)",
                  "x": xw, "w": w, "eps_f32": f32(1e-6),
                  "y": exact_tiny.rms(xw, w, f32(1e-6))})
    cases.append({"name": "layer_weighted_bias", "op": "layer",
                  "source": "Emily.Fast docs, layer_norm (weight and bias of shape {width})",
                  "x": xw, "w": w, "b": b, "eps_f32": f32(1e-5),
                  "y": exact_tiny.layer(xw, w, b, f32(1e-5))})
    cases.append({"name": "layer_big_eps", "op": "layer",
                  "source": "Emily.Fast docs, layer_norm (eps inside the square root)",
                  "x": xw, "w": w, "b": b, "eps_f32": 0.25,
                  "y": exact_tiny.layer(xw, w, b, 0.25)})
    # Emily.Fast docs, `rope` example: x = iota({1, 1, 4, 8}) (4 positions of
    # an 8-wide head), offset 0, dims 8, default base 10000 and scale 1; both
    # pair layouts; and the `rope_with_freqs` example table [1, .1, .01, .001].
    xs = [[float(r * 8 + j) for j in range(8)] for r in range(4)]
    for trad in (False, True):
        cases.append({"name": f"rope_doc_example_{'interleaved' if trad else 'split'}",
                      "op": "rope", "source": "Emily.Fast docs, rope, Examples",
                      "x": xs, "dims": 8, "traditional": trad, "base": 10000.0,
                      "scale": 1.0, "offset": 0, "freqs": None,
                      "y": [exact_tiny.rope_row_complex(row, p, 8, trad, 10000.0, 1.0)
                            for p, row in enumerate(xs)]})
    fr = [f32(1.0), f32(0.1), f32(0.01), f32(0.001)]
    cases.append({"name": "rope_with_freqs_doc_example", "op": "rope",
                  "source": "Emily.Fast docs, rope_with_freqs, Examples",
                  "x": xs, "dims": 8, "traditional": False, "base": 10000.0, "scale": 1.0,
                  "offset": 0, "freqs": fr,
                  "y": [exact_tiny.rope_row_complex(row, p, 8, False, 10000.0, 1.0, fr)
                        for p, row in enumerate(xs)]})
    cases.append({"name": "rope_offset_scale_partial_dims", "op": "rope",
                  "source": "Emily.Fast docs, rope (offset, scale, dims)",
                  "x": xs, "dims": 4, "traditional": False, "base": 500.0, "scale": 0.5,
                  "offset": 37, "freqs": None,
                  "y": [exact_tiny.rope_row_complex(row, 37 + p, 4, False, 500.0, 0.5)
                        for p, row in enumerate(xs)]})
    with open(os.path.join(HERE, "hand_cases.json"), "w") as f:
        json.dump({"generated_by": "tests/golden/make_golden.py (oracle/exact_tiny.py)",
                   "cases": cases}, f, indent=1)


if __name__ == "__main__":
    main()
