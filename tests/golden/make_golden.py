"""Write the stored expected values under tests/golden/.

Calls only the float64 oracle (and closed forms written out below); never the
HIP library.  Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gen.inputs import page_ce_tiny, page_kl_tiny  # noqa: E402

# Gradient columns stored for every row of the KL page case (plus the
# teacher ids of that row).
KL_COLS = [0, 1, 511, 1023]


def ce_page():
    c = page_ce_tiny()
    loss, lse, grad = oracle.ce(c["logits"], c["labels"], rng=c["rng"], scale=c["scale"])
    return {
        "source": "aprender-train 0.36.0, entrenar/autograd/wgpu_cross_entropy.rs, "
                  "test test_fused_ce_matches_naive: 4 tokens, vocabulary 8, logits "
                  "sin(0.3 i), labels [2, 5, 1, 7], every token in the loss; backward "
                  "scale 1/(loss_end - loss_start) = 1/4 as in backward()",
        "inputs": "gen.inputs.page_ce_tiny()",
        "expected_by": "oracle.ce (float64)",
        "seq_len": 4, "loss_start": 0, "loss_end": 4, "scale": c["scale"],
        "labels": c["labels"].tolist(),
        "loss": loss.tolist(),
        "mean_loss": float(loss.sum() / 4),
        "lse": lse.tolist(),
        "grad": grad.tolist(),
    }


def kl_page():
    c = page_kl_tiny()
    loss, lse, grad = oracle.kl(c["logits"], c["ids"], c["probs"], coef=c["coef"])
    picks = []
    for t in range(grad.shape[0]):
        cols = sorted(set(KL_COLS) | set(int(i) for i in c["ids"][t]))
        picks.append({"row": t, "cols": cols, "grad": [float(grad[t, j]) for j in cols]})
    return {
        "source": "cortiq-engine 0.8.21, src/gpu_wgpu/train_head.rs, test "
                  "head_kl_matches_host, for its shapes only: V=1024, hs=256, 45 tokens, "
                  "k=16, coef = gscale/total = 256/45; the values are seeded draws of "
                  "gen.inputs (N(0, 1/hs) head, N(0, 1) hidden rows, distinct uniform ids, "
                  "softmax(N(0, 1)) probabilities), the logits handed over directly as "
                  "the f64 product of the f16-rounded head and hidden rows",
        "inputs": "gen.inputs.page_kl_tiny()",
        "expected_by": "oracle.kl (float64)",
        "coef": c["coef"],
        "loss": loss.tolist(),
        "lse": lse.tolist(),
        "grad_samples": picks,
    }


def closed_forms():
    """Cases whose expected values follow from the formulas by hand."""
    cases = []
    # CE on a constant row: loss = ln V, gradient scale*(1/V - [j = label]).
    for V in (8, 512, 32000):
        cases.append({"op": "ce", "V": V, "row_value": 1.25, "label": V - 1, "scale": 0.5,
                      "loss": math.log(V), "grad_label": 0.5 * (1.0 / V - 1.0),
                      "grad_other": 0.5 / V})
    # KL, constant student, uniform teacher over k distinct ids (k a power of
    # two, so p = 1/k exactly): KL = ln(V/k).
    for V, k in ((1024, 16), (32000, 64), (151936, 256)):
        cases.append({"op": "kl", "V": V, "k": k, "row_value": -2.0, "coef": 1.0,
                      "loss": math.log(V / k), "grad_on_support": 1.0 / V - 1.0 / k,
                      "grad_off_support": 1.0 / V})
    # Top-k of a fixed row with ties and signed zeros: value desc, id asc.
    row = [0.5, -0.0, 2.0, 0.5, 0.0, 2.0, -1.0, 0.5]
    ids = [2, 5, 0, 3, 7, 1, 4]
    vals = [row[i] for i in ids]
    z = sum(math.exp(v - vals[0]) for v in vals)
    cases.append({"op": "topk", "row": row, "k": 7, "ids": ids,
                  "probs": [math.exp(v - vals[0]) / z for v in vals]})
    return {"source": "closed forms of the CE and KL definitions (aprender-train "
                      "wgpu_cross_entropy.rs module doc; cortiq-engine train_head.rs module "
                      "doc) and the top-k order (value descending, id ascending)",
            "cases": cases}


def main():
    for name, fn in (("ce_page_tiny.json", ce_page), ("kl_page_tiny.json", kl_page),
                     ("closed_forms.json", closed_forms)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fn(), f, indent=1)
            f.write("\n")
        print("wrote", name)


if __name__ == "__main__":
    main()
