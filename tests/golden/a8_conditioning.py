"""Conditioning of the W8A8 backbone at the two-camera long-context workload,
measured on the float64 oracle alone: every activation row is perturbed by a
relative 6e-8 (float32 rounding) before it is quantised, and the hidden state
after the final norm is compared with the unperturbed one. Per-token fp8
requantisation in every Linear turns such perturbations into whole-code steps
that later layers amplify, so this deviation is a floor for any float32
implementation of the model against the float64 oracle. Writes
tests/golden/a8_conditioning.json (several minutes on 8 cores):

    python tests/golden/a8_conditioning.py
"""

import dataclasses
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import fp8, llm, ops  # noqa: E402
from oracle.io import Weights, to_f64  # noqa: E402
from synth import get_config, make_inputs, make_weights  # noqa: E402

REL = 6e-8
SEED = 0


def hidden(cfg, W, x, perturb):
    orig = llm.fake_quant_act_rows
    if perturb:
        rng = np.random.default_rng(SEED)
        llm.fake_quant_act_rows = lambda t: orig(t * (1 + REL * rng.uniform(-1, 1, t.shape)))
    try:
        h = x
        for l in range(cfg.layers):
            h = llm.block(h, W, f"llm.{l}.", cfg.block)
        return ops.rmsnorm(h, W["llm.final_norm"], cfg.block.eps)
    finally:
        llm.fake_quant_act_rows = orig


def main():
    cfg = get_config(5)
    cfg = cfg.replace(block=dataclasses.replace(cfg.block, a8="fp8"))
    Wt = make_weights(cfg)
    Wt.generate_all(threads=8)
    W = Weights(Wt)
    x = to_f64(make_inputs(cfg)["text"])
    a = hidden(cfg, W, x, False)
    b = hidden(cfg, W, x, True)
    dev = float(np.linalg.norm(b - a) / np.linalg.norm(a))
    out = {"workload": cfg.name + " backbone, W8A8", "perturbation_rel": REL, "seed": SEED,
           "hidden_rel_l2_deviation": dev,
           "source": "tests/golden/a8_conditioning.py (float64 oracle only)"}
    path = os.path.join(ROOT, "tests", "golden", "a8_conditioning.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
