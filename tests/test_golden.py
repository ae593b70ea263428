"""The oracle against the stored fixtures under tests/golden/ (CPU only).

closed_forms.json holds values derived by hand from the definitions; the two
page fixtures hold oracle values on the inputs of the pages' own tests and
guard against an unnoticed change of the oracle's arithmetic."""
import json
import os

import numpy as np

import oracle
from gen.inputs import page_ce_tiny, page_kl_tiny

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_oracle_closed_forms():
    for c in load("closed_forms.json")["cases"]:
        if c["op"] == "ce":
            V = c["V"]
            x = np.full((1, V), c["row_value"], dtype=np.float32)
            loss, _, g = oracle.ce(x, [c["label"]], scale=c["scale"])
            assert abs(loss[0] - c["loss"]) < 1e-12
            assert abs(g[0, c["label"]] - c["grad_label"]) < 1e-15
            assert abs(g[0, 0] - c["grad_other"]) < 1e-15
        elif c["op"] == "kl":
            V, k = c["V"], c["k"]
            x = np.full((1, V), c["row_value"], dtype=np.float32)
            ids = (np.arange(k, dtype=np.uint32) * 7 + 3)[None, :]
            p = np.full((1, k), 1.0 / k, dtype=np.float32)
            loss, _, g = oracle.kl(x, ids, p, coef=c["coef"])
            assert abs(loss[0] - c["loss"]) < 1e-12
            assert abs(g[0, 3] - c["grad_on_support"]) < 1e-15
            assert abs(g[0, 4] - c["grad_off_support"]) < 1e-15
        elif c["op"] == "topk":
            row = np.array([c["row"]], dtype=np.float32)
            ids, probs = oracle.topk(row, c["k"])
            assert ids[0].tolist() == c["ids"]
            np.testing.assert_allclose(probs[0], c["probs"], rtol=1e-15)


def test_oracle_reproduces_ce_page_fixture():
    g = load("ce_page_tiny.json")
    c = page_ce_tiny()
    assert c["labels"].tolist() == g["labels"]
    loss, lse, grad = oracle.ce(c["logits"], c["labels"], rng=c["rng"], scale=c["scale"])
    np.testing.assert_allclose(loss, g["loss"], rtol=1e-15)
    np.testing.assert_allclose(lse, g["lse"], rtol=1e-15)
    np.testing.assert_allclose(grad, g["grad"], rtol=1e-14, atol=1e-18)


def test_oracle_reproduces_kl_page_fixture():
    g = load("kl_page_tiny.json")
    c = page_kl_tiny()
    loss, lse, grad = oracle.kl(c["logits"], c["ids"], c["probs"], coef=c["coef"])
    np.testing.assert_allclose(loss, g["loss"], rtol=1e-14)
    np.testing.assert_allclose(lse, g["lse"], rtol=1e-15)
    for s in g["grad_samples"]:
        np.testing.assert_allclose(grad[s["row"], s["cols"]], s["grad"], rtol=1e-13, atol=1e-18)
