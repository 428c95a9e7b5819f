"""Writes error_study_fig2.json: the synthetic analogue of the simulated
NVFP4 quantization study in "Four Over Six" sec. 2.2 (Fig. 2), computed by
the CPU oracle only.

The page measures word-level perplexity of a trained model; with no model
or dataset here, the measure is the relative squared error of the
dequantized tensor, sum((out - x)^2) / sum(x^2) in float64, on seeded
tensors shaped like the workloads' activations, weights and gradients.

  nvfp4          RTN6 NVFP4 (both error sources)
  scale_hp       block scale kept in fp32 (no E4M3 rounding)
  value_hp       scaled values kept in fp32 (no FP4 rounding)
  four_over_six  NVFP4 with the 4/6 block choice (for comparison)
  threshold      scaled values t rounded to FP4 only when |t| < x, for x in
                 0, 0.25, ..., 6.5 (x = 0: nothing rounded; x = 6.5 exceeds
                 every scaled value, i.e. plain NVFP4)

    python tests/golden/make_error_study.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synthetic as S  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "error_study_fig2.json")
SAMPLES = {"c1": (256, 1024), "c2": (1024, 4096), "c3": (1024, 4096), "c4": (512, 4096)}
THRESHOLDS = [0.25 * i for i in range(27)]


def rel_err(out, x_bits):
    y = S.bf16_bits_to_f32(x_bits).astype(np.float64)
    return float(((out.astype(np.float64) - y) ** 2).sum() / (y * y).sum())


def study(wl):
    x = S.gen(wl, *SAMPLES[wl])
    q = O.nvfp4_quantize(x, O.FOUR_OVER_SIX)
    d46 = O.dequantize(0, q["codes"], q["scales"], q["alpha"], *x.shape)
    return {
        "shape": list(x.shape),
        "nvfp4": rel_err(O.nvfp4_simulate(x, O.SIM_NVFP4), x),
        "scale_hp": rel_err(O.nvfp4_simulate(x, O.SIM_SCALE_HP), x),
        "value_hp": rel_err(O.nvfp4_simulate(x, O.SIM_VALUE_HP), x),
        "four_over_six": rel_err(d46, x),
        "threshold": [[t, rel_err(O.nvfp4_simulate(x, O.SIM_THRESHOLD, t), x)] for t in THRESHOLDS],
    }


def main():
    O.build()
    res = {"source": "Four Over Six, sec. 2.2, Fig. 2 (synthetic analogue)",
           "metric": "sum((out - x)^2) / sum(x^2), float64",
           "workloads": {wl: study(wl) for wl in SAMPLES}}
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
