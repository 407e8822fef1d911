"""Write workloads/sigma_table.json: mean overlap alpha as a function of sigma.

The Zipf-plus-Gaussian recipe sets target = draft + N(0, sigma^2); this script
measures alpha = mean over rows of sum_x min(p, q) (the acceptance probability
of the speculative-decoding blog, section 3) with the oracle's float64 softmax,
on the stored (rounded) logits, over a grid of sigma.  Common random numbers
across the grid keep the curve monotone.  Only the oracle computes here.

    python oracle/calibrate_sigma.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, _ROOT)

from oracle import softmax_rows, acceptance_probability  # noqa: E402
import workloads as W  # noqa: E402

SIGMAS = [0.02, 0.05, 0.08, 0.1, 0.15, 0.2, 0.25, 0.3, 0.35, 0.4, 0.45, 0.5, 0.6, 0.7,
          0.8, 0.9, 1.0, 1.2, 1.4, 1.6, 1.8, 2.0, 2.5, 3.0, 4.0]
ROWS = 16
CURVES = [(32000, 1.0, "f32"), (128256, 0.8, "bf16"), (152064, 1.0, "bf16"),
          (128256, 1.0, "bf16"), (4096, 1.0, "bf16"), (4096, 1.0, "f32"), (1000, 1.0, "f32")]


def curve(V: int, T: float, dtype: str, seed: int = 9000) -> tuple[list, list]:
    rng = W.philox(seed, V)
    d64 = W.zipf_rows(rng, ROWS, V)
    z = rng.standard_normal((ROWS, V))
    p, _, _ = softmax_rows(W.decode_f64(W.encode(d64, dtype), dtype), T)
    alphas = []
    for s in SIGMAS:
        q, _, _ = softmax_rows(W.decode_f64(W.encode(d64 + s * z, dtype), dtype), T)
        alphas.append(float(acceptance_probability(p, q).mean()))
    return SIGMAS, alphas


def main() -> None:
    out = {"rows_per_point": ROWS, "note": "alpha = mean_rows sum_x min(p,q), oracle softmax",
           "curves": {}}
    for V, T, dtype in CURVES:
        s, a = curve(V, T, dtype)
        out["curves"][f"V{V}_T{T:g}_{dtype}"] = {"sigma": s, "alpha": a}
        print(V, T, dtype, " ".join(f"{x:.2f}:{y:.3f}" for x, y in zip(s, a)))
    with open(os.path.join(_ROOT, "workloads", "sigma_table.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
