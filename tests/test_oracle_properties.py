"""Property-based pins of the oracle (hypothesis, CPU): for random rows,
teacher supports and partitions of the vocabulary into slices, the sliced
KL (per-slice statistics, merge, slice gradients) reproduces the separately
written C KL routine; the KL is never negative; CE equals KL with a unit
target; top-k agrees with a full lexicographic sort."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None)


@st.composite
def kl_case(draw):
    V = draw(st.integers(2, 300))
    n = draw(st.integers(1, 4))
    k = draw(st.integers(1, min(V, 24)))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    x = (rng.normal(size=(n, V)) * draw(st.sampled_from([0.5, 2.0, 8.0]))).astype(np.float32)
    ids = np.stack([rng.choice(V, size=k, replace=False) for _ in range(n)]).astype(np.uint32)
    p = rng.random((n, k)) + 1e-3
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    cuts = sorted(set(draw(st.lists(st.integers(1, V - 1), max_size=6)))) if V > 1 else []
    bounds = [0] + cuts + [V]
    widths = [b - a for a, b in zip(bounds[:-1], bounds[1:])]
    bf16 = draw(st.booleans())
    if bf16:
        u = x.view(np.uint32).astype(np.uint64)
        x = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return x, ids, p, list(zip(bounds[:-1], widths))


@SETTINGS
@given(kl_case(), st.floats(0.01, 4.0))
def test_sliced_kl_equals_whole_row_kl(case, coef):
    x, ids, p, cuts = case
    parts = [oracle.kl_slice_part(x[:, o:o + w], o, ids, p) for o, w in cuts]
    loss, lse = oracle.kl_slice_merge(parts)
    wl, wlse, wg = oracle.kl(x, ids, p, coef=coef)
    np.testing.assert_allclose(loss, wl, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, wlse, rtol=1e-12, atol=1e-12)
    g = np.concatenate([oracle.kl_slice_bwd(x[:, o:o + w], o, ids, p, wlse, coef=coef)
                        for o, w in cuts], axis=1)
    np.testing.assert_allclose(g, wg, rtol=1e-10, atol=1e-15)
    assert (wl >= -1e-12).all()


@SETTINGS
@given(st.integers(1, 500), st.integers(0, 2 ** 31 - 1), st.floats(0.01, 2.0))
def test_ce_is_kl_with_unit_target(V, seed, scale):
    rng = np.random.default_rng(seed)
    x = (rng.normal(size=(3, V)) * 3).astype(np.float32)
    lab = rng.integers(0, V, size=3).astype(np.uint32)
    lc, sc, gc = oracle.ce(x, lab, scale=scale)
    lk, sk, gk = oracle.kl(x, lab[:, None], np.ones((3, 1), np.float32), coef=scale)
    np.testing.assert_allclose(lk, lc, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gk, gc, rtol=1e-13, atol=1e-16)


@SETTINGS
@given(st.integers(1, 400), st.integers(0, 2 ** 31 - 1), st.data())
def test_topk_matches_full_sort(V, seed, data):
    k = data.draw(st.integers(1, V))
    rng = np.random.default_rng(seed)
    # few distinct values, signed zeros included: ties are the common case
    vals = np.array([-2.0, -0.0, 0.0, 0.5, 1.0, 3.0], dtype=np.float32)
    x = vals[rng.integers(0, len(vals), size=(2, V))]
    ids, probs = oracle.topk(x, k)
    for r in range(2):
        key = x[r].astype(np.float64) + 0.0  # -0 == +0
        want = np.lexsort((np.arange(V), -key))[:k]
        assert np.array_equal(ids[r].astype(np.int64), want)
        assert abs(probs[r].sum() - 1.0) < 1e-12
