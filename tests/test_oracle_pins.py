"""Pins of the float64 oracle against facts it does not itself define:
closed forms, invariants, finite differences, brute force, and independent
library routines (scipy, torch autograd).  CPU only."""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(12345)


def rows_f32(n, V, sigma=2.0, rng=RNG):
    return (rng.normal(size=(n, V)) * sigma).astype(np.float32)


def f32_to_bf16_bits(x):
    """Round-to-nearest-even float32 -> bf16 bit patterns (numpy uint16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------- lse

def test_lse_constant_row_closed_form():
    for V in (1, 7, 512, 32000):
        for c in (0.0, -3.5, 17.25):
            row = np.full(V, c, dtype=np.float32)
            assert abs(oracle.row_lse(row) - (c + math.log(V))) < 1e-12


def test_lse_matches_scipy_and_bounds():
    x = rows_f32(20, 1000, 3.0)
    for r in x:
        got = oracle.row_lse(r)
        want = scipy.special.logsumexp(r.astype(np.float64))
        assert abs(got - want) <= 1e-13 * abs(want) + 1e-13
        m = float(r.max())
        assert m <= got <= m + math.log(r.size) + 1e-12


def test_bf16_widening_is_exact():
    # bf16 bit patterns with known values: 1.0, -2.0, 0.5, 3.140625, -0.0
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x4049, 0x8000], dtype=np.uint16)
    vals = [1.0, -2.0, 0.5, 3.140625, -0.0]
    for b, v in zip(bits, vals):
        assert oracle.row_lse(np.array([b], dtype=np.uint16)) == v
    x = rows_f32(4, 300)
    b = f32_to_bf16_bits(x)
    for i in range(4):
        want = scipy.special.logsumexp(bf16_bits_to_f64(b[i]))
        assert abs(oracle.row_lse(b[i]) - want) < 1e-12


def test_lse_minus_inf_entries():
    row = np.array([-np.inf, 0.0, -np.inf, math.log(3.0)], dtype=np.float32)
    want = math.log(1.0 + math.exp(float(np.float32(math.log(3.0)))))
    assert abs(oracle.row_lse(row) - want) < 1e-12


# ----------------------------------------------------------------- CE

def test_ce_loss_matches_torch_cross_entropy():
    x = rows_f32(32, 777, 3.0)
    lab = RNG.integers(0, 777, size=32)
    loss, lse, _ = oracle.ce(x, lab, want_grad=False)
    want = F.cross_entropy(torch.from_numpy(x).double(), torch.from_numpy(lab).long(),
                           reduction="none").numpy()
    np.testing.assert_allclose(loss, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(x.astype(np.float64), axis=1),
                               rtol=1e-13)


def test_ce_uniform_row_is_ln_V():
    for V in (2, 10, 32000):
        x = np.full((3, V), 1.5, dtype=np.float32)
        loss, _, g = oracle.ce(x, [0, V // 2, V - 1], scale=1.0)
        np.testing.assert_allclose(loss, math.log(V), rtol=1e-14)
        # gradient: 1/V everywhere, 1/V - 1 at the label
        assert abs(g[1, V // 2] - (1.0 / V - 1.0)) < 1e-14
        assert abs(g[1, 0] - 1.0 / V) < 1e-14 or V // 2 == 0


def test_ce_dominant_label_loss_near_zero():
    x = np.zeros((1, 100), dtype=np.float32)
    x[0, 42] = 60.0
    loss, _, g = oracle.ce(x, [42])
    # loss = ln(1 + 99 e^-60) ~ 8.7e-25, below float64 resolution at lse = 60:
    # the definition lse - s_label is exact to a few ulp of lse.
    assert 0.0 <= loss[0] < 1e-14
    assert abs(loss[0] - 99 * math.exp(-60.0)) < 4 * np.spacing(60.0)
    assert abs(g[0, 42]) < 1e-20 and abs(g[0, 0] - math.exp(-60.0)) < 1e-40


def test_ce_grad_matches_torch_autograd():
    x = rows_f32(16, 333, 2.5)
    lab = RNG.integers(0, 333, size=16)
    scale = 1.0 / 16
    _, _, g = oracle.ce(x, lab, scale=scale)
    t = torch.from_numpy(x).double().requires_grad_()
    (F.cross_entropy(t, torch.from_numpy(lab).long(), reduction="sum") * scale).backward()
    np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-12, atol=1e-16)


def test_ce_grad_finite_differences():
    # Central differences of the oracle's own loss with exact float32 steps.
    h = 2.0 ** -12
    x = rows_f32(3, 9, 1.5)
    lab = np.array([0, 4, 8])
    _, _, g = oracle.ce(x, lab, scale=1.0)
    for i in range(3):
        for j in range(9):
            xp = x[i:i + 1].copy(); xp[0, j] += np.float32(h)
            xm = x[i:i + 1].copy(); xm[0, j] -= np.float32(h)
            dp = float(xp[0, j]) - float(x[i, j]); dm = float(x[i, j]) - float(xm[0, j])
            assert dp == h and dm == h
            lp = oracle.ce(xp, lab[i:i + 1], want_grad=False)[0][0]
            lm = oracle.ce(xm, lab[i:i + 1], want_grad=False)[0][0]
            assert abs((lp - lm) / (2 * h) - g[i, j]) < 1e-7


def test_ce_grad_rows_sum_to_zero_and_scale_applies():
    x = rows_f32(8, 1000)
    lab = RNG.integers(0, 1000, size=8)
    _, _, g1 = oracle.ce(x, lab, scale=1.0)
    _, _, g3 = oracle.ce(x, lab, scale=0.125)
    assert np.abs(g1.sum(axis=1)).max() < 1e-13
    np.testing.assert_allclose(g3, 0.125 * g1, rtol=1e-15, atol=0)


def test_ce_loss_range_masks_rows():
    x = rows_f32(12, 50)
    lab = RNG.integers(0, 50, size=12)
    full_loss, full_lse, full_g = oracle.ce(x, lab, scale=0.5)
    rng = (5, 1, 3)  # rows with r mod 5 in {1, 2}
    loss, lse, g = oracle.ce(x, lab, rng=rng, scale=0.5)
    for r in range(12):
        if 1 <= r % 5 < 3:
            assert loss[r] == full_loss[r] and lse[r] == full_lse[r]
            assert np.array_equal(g[r], full_g[r])
        else:
            assert loss[r] == 0.0 and lse[r] == 0.0 and not g[r].any()
    # row_index shifts the range test: rows 0..3 treated as global rows 5..8
    l2, _, _ = oracle.ce(x[:4], lab[:4], rng=rng, row_index=np.arange(5, 9), want_grad=False)
    assert l2[0] == 0.0 and l2[1] == full_loss[1] and l2[2] == full_loss[2] and l2[3] == 0.0


def test_ce_page_test_mean_loss():
    """aprender-train wgpu_cross_entropy.rs test: the page's own float32 CPU
    reference of the mean loss agrees with the oracle's mean (the page's
    tolerance, 1e-4), and the mean is taken over the range count."""
    from gen.inputs import page_ce_tiny
    c = page_ce_tiny()
    x, lab = c["logits"], c["labels"]
    # the page's reference, in float32 as printed there
    cpu = np.float32(0.0)
    for r in range(4):
        mx = np.float32(-np.inf)
        for v in x[r]:
            mx = max(mx, v)
        se = np.float32(0.0)
        for v in x[r]:
            se = np.float32(se + np.exp(np.float32(v - mx)))
        cpu = np.float32(cpu + (-x[r, lab[r]] + np.float32(mx + np.log(se))))
    cpu = cpu / np.float32(4)
    loss, _, _ = oracle.ce(x, lab, rng=c["rng"], want_grad=False)
    assert abs(loss.sum() / 4 - float(cpu)) < 1e-4


# ------------------------------------------- CE split: backward from lse, mean

def test_ce_bwd_constant_rows_closed_form():
    """Row r constant c_r with its saved lse c_r + ln V (rounded to float32):
    every softmax entry is 1/V, so g = scale (1/V - [j = label]).  The rows
    differ, so a logsumexp taken from the wrong row fails."""
    V, n = 16, 6
    c = np.array([-3.0, -1.5, 0.0, 0.75, 2.0, 5.5], dtype=np.float32)
    x = np.repeat(c[:, None], V, axis=1)
    lab = np.array([0, 3, 15, 7, 1, 9])
    lse = (c.astype(np.float64) + math.log(V)).astype(np.float32)
    g = oracle.ce_bwd(x, lab, lse, scale=0.25)
    want = np.full((n, V), 0.25 / V)
    want[np.arange(n), lab] -= 0.25
    # lse is float32: p = exp(c - fl(c + ln V)) = (1/V)(1 + O(2^-24 |lse|))
    np.testing.assert_allclose(g, want, rtol=0, atol=0.25 / V * 1e-6)


def test_ce_bwd_matches_scipy_softmax():
    """With the correctly rounded float32 logsumexp of each row (scipy), the
    gradient is scale (softmax(row) - one_hot) from scipy, up to that
    rounding."""
    x = rows_f32(5, 3000)
    lab = RNG.integers(0, 3000, size=5)
    lse64 = scipy.special.logsumexp(x.astype(np.float64), axis=1)
    g = oracle.ce_bwd(x, lab, lse64.astype(np.float32), scale=0.5)
    sm = scipy.special.softmax(x.astype(np.float64), axis=1)
    sm[np.arange(5), lab] -= 1.0
    err = np.abs(g - 0.5 * sm)
    tol = 0.5 * np.abs(sm) * (np.abs(lse64)[:, None] * 2.0**-23 + 1e-14)
    assert (err <= tol + 1e-300).all()


def test_ce_bwd_lse_shift_scales_softmax_part():
    """Raising the saved lse by 1 divides the softmax part exp(s - lse) by e
    and leaves the one-hot part: g + scale onehot scales by exp(-1)."""
    x = rows_f32(3, 200)
    lab = np.array([5, 0, 199])
    lse = np.array([2.5, -1.0, 7.0], dtype=np.float32)  # lse + 1 exact in float32
    g0 = oracle.ce_bwd(x, lab, lse, scale=2.0)
    g1 = oracle.ce_bwd(x, lab, lse + np.float32(1.0), scale=2.0)
    oh = np.zeros_like(g0)
    oh[np.arange(3), lab] = 2.0
    # adding the one-hot back at the label cancels: one ulp of scale absolute
    np.testing.assert_allclose(g1 + oh, (g0 + oh) * math.exp(-1.0), rtol=1e-14,
                               atol=2.0 * 2.0**-52)


def test_ce_bwd_range_and_bf16():
    """Rows outside the range are zero; bf16 rows are read through the exact
    widening (same result as their float32 widening)."""
    x = rows_f32(10, 64)
    b = f32_to_bf16_bits(x)
    xw = bf16_bits_to_f64(b).astype(np.float32)
    lab = RNG.integers(0, 64, size=10)
    lse = np.linspace(1.0, 4.0, 10).astype(np.float32)
    rng = (4, 1, 3)
    gb = oracle.ce_bwd(b, lab, lse, rng=rng, scale=1.0)
    gw = oracle.ce_bwd(xw, lab, lse, rng=rng, scale=1.0)
    assert np.array_equal(gb, gw)
    for r in range(10):
        if 1 <= r % 4 < 3:
            assert gb[r].any()
        else:
            assert not gb[r].any()


def test_loss_mean_hand_cases():
    """The mean loss sums every row and divides by the rows in the range
    (read_loss); values worked by hand."""
    l8 = np.arange(1, 9, dtype=np.float32)  # sum 36
    assert oracle.loss_mean(l8) == 4.5
    assert oracle.loss_mean(l8, (4, 1, 3)) == 9.0     # rows 1, 2, 5, 6 in range
    assert oracle.loss_mean(l8, (8, 2, 5)) == 12.0    # rows 2, 3, 4
    assert oracle.loss_mean(l8, (8, 3, 3)) == 0.0     # empty range
    l10 = np.arange(1, 11, dtype=np.float32)  # sum 55; rows 1, 2, 5, 6, 9
    assert oracle.loss_mean(l10, (4, 1, 3)) == 11.0
    assert oracle.loss_mean(np.zeros(0, dtype=np.float32)) == 0.0


# ----------------------------------------------------------------- KL

def renorm_probs(n, k, sigma=1.5, rng=RNG):
    z = rng.normal(size=(n, k)) * sigma
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def distinct(n, V, k, rng=RNG):
    return np.stack([rng.choice(V, size=k, replace=False) for _ in range(n)]).astype(np.uint32)


def dyadic_probs(n, k, rng=RNG):
    """Probabilities that are multiples of 2^-10 and sum to exactly 1 in
    float32 and float64."""
    out = np.empty((n, k), dtype=np.float32)
    for i in range(n):
        cuts = np.sort(rng.choice(np.arange(1, 1024), size=k - 1, replace=False))
        c = np.diff(np.concatenate([[0], cuts, [1024]]))
        out[i] = c / 1024.0
    assert (out.astype(np.float64).sum(axis=1) == 1.0).all()
    return out


def kl_autograd(x, ids, p, coef):
    t = torch.from_numpy(x).double().requires_grad_()
    logp = F.log_softmax(t, dim=1).gather(1, torch.from_numpy(ids.astype(np.int64)))
    per_row = F.kl_div(logp, torch.from_numpy(p).double(), reduction="none").sum(dim=1)
    (per_row.sum() * coef).backward()
    return per_row.detach().numpy(), t.grad.numpy()


def test_kl_matches_torch_kl_div_and_autograd():
    n, V, k = 10, 500, 16
    x = rows_f32(n, V)
    ids = distinct(n, V, k)
    p = dyadic_probs(n, k)
    coef = 1024.0 / n
    loss, _, g = oracle.kl(x, ids, p, coef=coef)
    want_loss, want_g = kl_autograd(x, ids, p, coef)
    np.testing.assert_allclose(loss, want_loss, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g, want_g, rtol=1e-11, atol=1e-14)


def test_kl_gradient_uses_probs_as_given():
    """With sum(p) != 1 the oracle applies p_S - p_T literally (no
    renormalisation); the exact derivative of the loss is then
    sum(p) p_S - p_T, so the two differ by coef (1 - sum p) p_S."""
    n, V, k = 4, 300, 12
    x = rows_f32(n, V)
    ids = distinct(n, V, k)
    p = renorm_probs(n, k) * np.float32(0.9)
    _, _, g = oracle.kl(x, ids, p, coef=2.0)
    _, want_g = kl_autograd(x, ids, p, 2.0)
    ps = scipy.special.softmax(x.astype(np.float64), axis=1)
    mass = p.astype(np.float64).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(g, want_g + 2.0 * (1.0 - mass) * ps, rtol=1e-11, atol=1e-14)


def test_kl_nonnegative():
    n, V, k = 50, 200, 8
    loss, _, _ = oracle.kl(rows_f32(n, V, 4.0), distinct(n, V, k), renorm_probs(n, k, 3.0),
                           want_grad=False)
    assert (loss >= 0).all()


def test_kl_uniform_closed_form():
    for V, k in ((64, 1), (64, 8), (1000, 64)):
        x = np.full((2, V), -0.75, dtype=np.float32)
        ids = distinct(2, V, k)
        p = np.full((2, k), 1.0 / k, dtype=np.float32)
        loss, _, _ = oracle.kl(x, ids, p, want_grad=False)
        # p_q = fl32(1/k), so the exact value carries its rounding
        pq = float(np.float32(1.0 / k))
        want = k * pq * (math.log(pq) + math.log(V))
        np.testing.assert_allclose(loss, want, rtol=1e-13)
        if k in (1, 8, 64):  # powers of two: 1/k exact, KL = ln(V/k)
            np.testing.assert_allclose(loss, math.log(V / k), rtol=1e-13)


def test_kl_teacher_equal_to_student_on_support():
    n, V, k = 6, 300, 20
    x = rows_f32(n, V)
    ids = distinct(n, V, k)
    ps = scipy.special.softmax(x.astype(np.float64), axis=1)
    sup = np.take_along_axis(ps, ids.astype(np.int64), axis=1)
    mass = sup.sum(axis=1)
    p = (sup / mass[:, None]).astype(np.float32)
    loss, _, _ = oracle.kl(x, ids, p, want_grad=False)
    # exact with the float32-rounded probabilities:
    pd = p.astype(np.float64)
    want = (pd * (np.log(pd) - np.log(sup))).sum(axis=1)
    np.testing.assert_allclose(loss, want, rtol=1e-10, atol=1e-13)
    # and close to the closed form -ln(sum of p_S on the support)
    np.testing.assert_allclose(loss, -np.log(mass), rtol=1e-5)


def test_kl_student_minus_inf_off_support_is_zero():
    V, k = 40, 5
    x = np.full((1, V), -np.inf, dtype=np.float32)
    ids = np.array([[3, 7, 11, 20, 39]], dtype=np.uint32)
    vals = np.array([0.5, -1.0, 2.0, 0.0, 1.25], dtype=np.float32)
    x[0, ids[0]] = vals
    p = scipy.special.softmax(vals.astype(np.float64)).astype(np.float32)
    loss, _, g = oracle.kl(x, ids, p, coef=1.0)
    ps = scipy.special.softmax(vals.astype(np.float64))
    want = (p.astype(np.float64) * (np.log(p.astype(np.float64)) - np.log(ps))).sum()
    assert abs(loss[0] - want) < 1e-15 and abs(loss[0]) < 1e-7
    off = np.setdiff1d(np.arange(V), ids[0])
    assert not g[0, off].any()


def test_kl_grad_finite_differences():
    h = 2.0 ** -12
    V, k = 10, 4
    x = rows_f32(2, V, 1.5)
    ids = np.array([[0, 3, 5, 9], [1, 2, 8, 4]], dtype=np.uint32)
    p = renorm_probs(2, k)
    _, _, g = oracle.kl(x, ids, p, coef=1.0)
    for i in range(2):
        for j in range(V):
            xp = x[i:i + 1].copy(); xp[0, j] += np.float32(h)
            xm = x[i:i + 1].copy(); xm[0, j] -= np.float32(h)
            lp = oracle.kl(xp, ids[i:i + 1], p[i:i + 1], want_grad=False)[0][0]
            lm = oracle.kl(xm, ids[i:i + 1], p[i:i + 1], want_grad=False)[0][0]
            assert abs((lp - lm) / (2 * h) - g[i, j]) < 1e-7


def test_kl_zero_prob_terms_and_row_sum():
    V = 64
    x = rows_f32(1, V)
    ids = np.array([[5, 9, 17]], dtype=np.uint32)
    p = np.array([[0.25, 0.0, 0.5]], dtype=np.float32)  # sums to 0.75 (used as given)
    loss, _, g = oracle.kl(x, ids, p, coef=2.0)
    l2, _, g2 = oracle.kl(x, ids[:, [0, 2]], p[:, [0, 2]], coef=2.0)
    assert loss[0] == l2[0]
    np.testing.assert_array_equal(g, g2)
    assert abs(g.sum() - 2.0 * (1 - 0.75)) < 1e-13


def test_kl_duplicate_ids_sum_their_probs():
    x = rows_f32(1, 30)
    _, _, g = oracle.kl(x, np.array([[4, 4]], dtype=np.uint32),
                        np.array([[0.25, 0.5]], dtype=np.float32), coef=1.0)
    ps = scipy.special.softmax(x[0].astype(np.float64))
    assert abs(g[0, 4] - (ps[4] - 0.75)) < 1e-15


def test_ce_equals_kl_with_unit_target():
    """The two oracle routines are written separately; with k=1 and p=1 the
    distillation KL is the cross-entropy."""
    x = rows_f32(7, 257)
    lab = RNG.integers(0, 257, size=7).astype(np.uint32)
    lc, sc, gc = oracle.ce(x, lab, rng=(7, 2, 6), scale=0.3)
    lk, sk, gk = oracle.kl(x, lab[:, None], np.ones((7, 1), np.float32), rng=(7, 2, 6),
                           coef=0.3)
    np.testing.assert_allclose(lk, lc, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(sk, sc)
    np.testing.assert_allclose(gk, gc, rtol=1e-14, atol=1e-17)


def test_kl_page_test_host_reference():
    """cortiq-engine train_head.rs head_kl_matches_host: its float64 host
    reference (loss and the 1/ntok-scaled logits gradient) at the page
    test's shapes, on seeded inputs."""
    from gen.inputs import page_kl_tiny
    c = page_kl_tiny()
    x, ids, p = c["logits"], c["ids"], c["probs"]
    ntok, V = x.shape
    loss, _, g = oracle.kl(x, ids, p, coef=1.0 / ntok)
    want_loss = np.zeros(ntok)
    want_d = np.zeros((ntok, V))
    for t in range(ntok):
        s = x[t].astype(np.float64)
        mx = s.max()
        lse = mx + math.log(np.exp(s - mx).sum())
        d = np.exp(s - lse) / ntok
        for q in range(ids.shape[1]):
            pt = float(p[t, q])
            want_loss[t] += pt * (math.log(pt) - (s[ids[t, q]] - lse))
            d[ids[t, q]] -= pt / ntok
        want_d[t] = d
    rel = np.linalg.norm(loss - want_loss) / np.linalg.norm(want_loss)
    assert rel < 1e-12
    assert np.linalg.norm(g - want_d) / np.linalg.norm(want_d) < 1e-12


# ----------------------------------------------------------------- top-k

def brute_topk(vals64, k):
    ids = np.arange(vals64.size)
    order = np.lexsort((ids, -vals64))  # value desc, then id asc
    return order[:k]


@pytest.mark.parametrize("V,k", [(50, 1), (50, 7), (50, 50), (1000, 64), (4097, 300)])
def test_topk_brute_force_with_ties(V, k):
    rng = np.random.default_rng(V * 31 + k)
    x = (rng.integers(-6, 7, size=(8, V)) * 0.5).astype(np.float32)  # many ties
    ids, probs = oracle.topk(x, k)
    for i in range(8):
        v = x[i].astype(np.float64)
        np.testing.assert_array_equal(ids[i], brute_topk(v, k))
        sel = v[ids[i]]
        np.testing.assert_allclose(probs[i], scipy.special.softmax(sel), rtol=1e-14)
        assert abs(probs[i].sum() - 1.0) < 1e-14
        assert (np.diff(probs[i]) <= 0).all()


def test_topk_special_rows():
    V = 20
    ids, _ = oracle.topk(np.full((1, V), 3.0, np.float32), 5)
    np.testing.assert_array_equal(ids[0], [0, 1, 2, 3, 4])
    # -0 and +0 tie: lower id first
    row = np.array([[-0.0, 0.0, -0.0, -1.0]], dtype=np.float32)
    ids, probs = oracle.topk(row, 3)
    np.testing.assert_array_equal(ids[0], [0, 1, 2])
    np.testing.assert_allclose(probs[0], 1 / 3, rtol=1e-15)
    # -inf entries are chosen last, by id
    row = np.full((1, 6), -np.inf, dtype=np.float32)
    row[0, 4] = 1.0
    ids, probs = oracle.topk(row, 3)
    np.testing.assert_array_equal(ids[0], [4, 0, 1])
    np.testing.assert_array_equal(probs[0], [1.0, 0.0, 0.0])
    # k = V gives a full permutation and the full softmax
    x = rows_f32(1, 100)
    ids, probs = oracle.topk(x, 100)
    assert sorted(ids[0].tolist()) == list(range(100))
    sm = scipy.special.softmax(x[0].astype(np.float64))
    np.testing.assert_allclose(probs[0], sm[ids[0]], rtol=1e-13)


def test_topk_bf16_ties_follow_widened_values():
    x = rows_f32(6, 3000, 2.0)
    b = f32_to_bf16_bits(x)
    ids, probs = oracle.topk(b, 256)
    for i in range(6):
        v = bf16_bits_to_f64(b[i])
        np.testing.assert_array_equal(ids[i], brute_topk(v, 256))
        np.testing.assert_allclose(probs[i], scipy.special.softmax(v[ids[i]]), rtol=1e-13)


# ----------------------------------------------------------------- acc

def test_acc_bit_exact_float32_add():
    rng = np.random.default_rng(7)
    a = rng.normal(size=100000).astype(np.float32) * np.float32(1e3)
    b = rng.normal(size=100000).astype(np.float32) * np.float32(1e-3)
    special = np.array([np.inf, -np.inf, -0.0, 0.0, 1e-40, -1e-40, 3.4e38, 3.4e38,
                        1.0, 2.0 ** -24], dtype=np.float32)
    special_b = np.array([1.0, -5.0, -0.0, -0.0, 1e-40, 2e-40, 3.4e38, -3.4e38,
                          2.0 ** -24, 1.0], dtype=np.float32)
    a = np.concatenate([a, special]); b = np.concatenate([b, special_b])
    got = oracle.acc(a, b)
    with np.errstate(over="ignore"):
        want = a + b  # numpy float32 add: correctly rounded, an independent route
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ----------------------------------------------------------------- head

def head_case(n=4, V=48, hs=12, k=5, seed=3):
    r = np.random.default_rng(seed)
    x = r.normal(size=(n, hs))
    w = r.normal(size=(V, hs)) * 0.4
    ids = np.stack([r.choice(V, size=k, replace=False) for _ in range(n)])
    z = r.normal(size=(n, k)) * 1.5
    p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    return x, w, ids, p


def test_head_dx_is_the_gradient_of_the_mean_loss():
    """Central differences of sum_t loss_t / total in each hidden entry
    match dx (the teacher probabilities sum to 1 up to float32 rounding, so
    the literal p_S - p_T gradient is the derivative)."""
    x, w, ids, p = head_case()
    total, gscale = 7, 256.0
    _, dx = oracle.head_kl(x, w, ids, p, total, gscale)
    h = 1e-6
    for t in range(x.shape[0]):
        for i in range(x.shape[1]):
            xp = x.copy(); xp[t, i] += h
            xm = x.copy(); xm[t, i] -= h
            lp, _ = oracle.head_kl(xp, w, ids, p, total, gscale)
            lm, _ = oracle.head_kl(xm, w, ids, p, total, gscale)
            fd = (lp.sum() - lm.sum()) / (2 * h * total)
            assert abs(fd - dx[t, i]) < 1e-6 * max(1.0, abs(dx[t, i])), (t, i, fd, dx[t, i])


def test_head_zero_weights_closed_form():
    """W = 0: every logit is 0, the student is uniform: loss = sum_q p_q
    ln(p_q V), and dx = 0."""
    x, w, ids, p = head_case()
    V = w.shape[0]
    loss, dx = oracle.head_kl(x, np.zeros_like(w), ids, p, 4, 2.0)
    pf = p.astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(loss, (pf * np.log(pf * V)).sum(axis=1), rtol=1e-13)
    assert not dx.any()


def test_head_matches_the_row_kl_on_exact_logits():
    """With dyadic inputs whose products are exact in float32, the head's
    loss equals the C oracle's KL on those logits and dx equals that
    gradient times W over gscale: the two are written separately."""
    r = np.random.default_rng(9)
    n, V, hs, k = 5, 64, 8, 6
    x = r.integers(-4, 5, size=(n, hs)) / 4.0
    w = r.integers(-8, 9, size=(V, hs)) / 8.0
    ids = np.stack([r.choice(V, size=k, replace=False) for _ in range(n)])
    p = (r.dirichlet(np.ones(k), size=n)).astype(np.float32)
    s = (x @ w.T).astype(np.float32)
    assert np.array_equal(s.astype(np.float64), x @ w.T)
    total, gscale = 9, 64.0
    loss, dx = oracle.head_kl(x, w, ids, p, total, gscale)
    kloss, _, g = oracle.kl(s, ids.astype(np.uint32), p, coef=gscale / total)
    np.testing.assert_allclose(loss, kloss, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dx, (g @ w) / gscale, rtol=1e-12, atol=1e-15)


def _dyadic_head(seed, n, V, hs):
    """Hidden rows and head weights of small dyadic values: every product
    and every partial sum of a logit is exact in float32 (and in float64)."""
    r = np.random.default_rng(seed)
    x = r.integers(-4, 5, size=(n, hs)) / 4.0
    w = r.integers(-8, 9, size=(V, hs)) / 8.0
    return x, w


def test_head_topk_matches_the_row_topk_on_exact_logits():
    """With exact float32 logits the head's top-k equals the C oracle's
    top-k of those logits (a separately written routine: a qsort of the
    whole row with the tie rule); coarse dyadic values make ties common."""
    for seed, (n, V, hs, k) in enumerate([(6, 64, 8, 10), (4, 300, 5, 64), (3, 50, 2, 50)]):
        x, w = _dyadic_head(20 + seed, n, V, hs)
        s = (x @ w.T).astype(np.float32)
        assert np.array_equal(s.astype(np.float64), x @ w.T)
        ids, probs = oracle.head_topk(x, w, k)
        cids, cprobs = oracle.topk(s, k)
        np.testing.assert_array_equal(ids, cids)
        np.testing.assert_allclose(probs, cprobs, rtol=1e-13, atol=1e-300)


def test_head_topk_brute_force_and_invariants():
    """Against a brute force over every pair of columns (an id ranks ahead
    of another iff its logit is larger, or equal with a lower id); probs
    sum to 1, do not increase, and k = V gives the whole row's softmax."""
    x, w = _dyadic_head(31, 5, 40, 3)
    s = x @ w.T
    V = s.shape[1]
    for k in (1, 7, V):
        ids, probs = oracle.head_topk(x, w, k)
        for t in range(s.shape[0]):
            rank = [sum(1 for j in range(V) if s[t, j] > s[t, i] or (s[t, j] == s[t, i] and j < i))
                    for i in range(V)]
            want = [i for i in sorted(range(V), key=lambda i: rank[i])][:k]
            assert ids[t].tolist() == want
            assert abs(probs[t].sum() - 1.0) < 1e-14
            assert np.all(np.diff(probs[t]) <= 1e-18)
        if k == V:
            e = np.exp(s - s.max(axis=1, keepdims=True))
            sm = e / e.sum(axis=1, keepdims=True)
            np.testing.assert_allclose(probs, np.take_along_axis(sm, ids.astype(np.int64), 1),
                                       rtol=1e-13)


def test_head_topk_zero_weights_give_the_first_ids():
    """W = 0: every logit is 0, all tie, so the ids are 0..k-1 with equal
    probabilities 1/k."""
    x, w = _dyadic_head(32, 3, 20, 4)
    ids, probs = oracle.head_topk(x, np.zeros_like(w), 6)
    assert (ids == np.arange(6)).all()
    np.testing.assert_allclose(probs, 1.0 / 6, rtol=1e-15)


def test_round_half_is_round_to_nearest_even():
    """f16 by numpy's cast; bf16 ties go to the even pattern."""
    one = np.float32(1.0)
    tie = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8)], dtype=np.float32)
    np.testing.assert_array_equal(oracle.round_half(tie, "bf16"), [1.0, 1.0 + 2**-6, -1.0])
    assert oracle.round_half(np.float32(1.0 + 2.0**-11), "f16") == 1.0
    assert oracle.round_half(one, "bf16") == 1.0


# ------------------------------------------------ vocabulary slices (KL)

def _cuts(V, widths):
    offs = np.cumsum([0] + list(widths))
    assert offs[-1] == V
    return [(int(o), int(w)) for o, w in zip(offs[:-1], widths)]


def _sliced(x, ids, p, cuts, rng=None):
    parts = [oracle.kl_slice_part(x[:, o:o + w], o, ids, p, rng=rng) for o, w in cuts]
    return parts, oracle.kl_slice_merge(parts, rng=rng)


def test_kl_slices_merge_to_the_whole_row_kl():
    """Merged slice statistics give the whole-row KL and logsumexp of the C
    routine (written separately), for ragged cuts and a loss range; the
    slice gradients from that lse are the whole-row gradient's columns."""
    n, V, k = 9, 1000, 24
    x = rows_f32(n, V, 3.0)
    ids = distinct(n, V, k)
    p = renorm_probs(n, k)
    rng = (3, 1, 3)
    for widths in ((V,), (500, 500), (333, 367, 300), (1, 998, 1), (64,) * 15 + (40,)):
        cuts = _cuts(V, widths)
        _, (loss, lse) = _sliced(x, ids, p, cuts, rng=rng)
        wl, wlse, wg = oracle.kl(x, ids, p, rng=rng, coef=0.625)
        np.testing.assert_allclose(loss, wl, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, wlse, rtol=1e-13, atol=0)
        g = np.concatenate([oracle.kl_slice_bwd(x[:, o:o + w], o, ids, p, wlse, coef=0.625,
                                                rng=rng) for o, w in cuts], axis=1)
        np.testing.assert_allclose(g, wg, rtol=1e-12, atol=1e-16)


def test_kl_slices_bf16_merge_to_the_whole_row_kl():
    n, V, k = 4, 640, 32
    b = f32_to_bf16_bits(rows_f32(n, V))
    ids = distinct(n, V, k)
    p = renorm_probs(n, k)
    _, (loss, lse) = _sliced(b, ids, p, _cuts(V, (320, 320)))
    wl, wlse, _ = oracle.kl(b, ids, p, want_grad=False)
    np.testing.assert_allclose(loss, wl, rtol=1e-12)
    np.testing.assert_allclose(lse, wlse, rtol=1e-13)


def test_kl_slice_part_closed_forms():
    # constant slice, no teacher entry in it: a = c, z = width exactly, P = w = 0
    x = np.full((2, 50), 1.75, dtype=np.float32)
    ids = np.array([[0, 1], [2, 3]], dtype=np.uint32)
    p = np.full((2, 2), 0.5, dtype=np.float32)
    part = oracle.kl_slice_part(x, 100, ids, p)
    np.testing.assert_array_equal(part, [[1.75, 50.0, 0.0, 0.0]] * 2)
    # one teacher entry of probability 1 at the slice's maximum: w = 0, P = 1
    y = np.array([[0.0, 3.0, -1.0]], dtype=np.float32)
    part = oracle.kl_slice_part(y, 7, np.array([[8]], np.uint32), np.array([[1.0]], np.float32))
    assert part[0, 0] == 3.0 and part[0, 2] == 1.0 and part[0, 3] == 0.0
    assert abs(part[0, 1] - (1.0 + math.exp(-3.0) + math.exp(-4.0))) < 1e-15


def test_kl_slices_uniform_closed_form():
    """Uniform student over V, uniform teacher over k ids spread over three
    slices: KL = ln(V / k)."""
    V, k = 96, 8
    x = np.full((1, V), -2.0, dtype=np.float32)
    ids = np.array([[0, 5, 31, 32, 40, 63, 64, 95]], dtype=np.uint32)
    p = np.full((1, k), 1.0 / k, dtype=np.float32)
    _, (loss, lse) = _sliced(x, ids, p, _cuts(V, (32, 32, 32)))
    assert abs(loss[0] - math.log(V / k)) < 1e-13
    assert abs(lse[0] - (-2.0 + math.log(V))) < 1e-13


def test_kl_slices_unit_target_is_the_cross_entropy():
    """k = 1, p = 1 over slices gives the C cross-entropy routine's loss and
    gradient."""
    n, V = 6, 301
    x = rows_f32(n, V)
    lab = RNG.integers(0, V, size=n).astype(np.uint32)
    one = np.ones((n, 1), np.float32)
    cuts = _cuts(V, (100, 101, 100))
    _, (loss, lse) = _sliced(x, lab[:, None], one, cuts)
    wl, wlse, wg = oracle.ce(x, lab, scale=0.5)
    np.testing.assert_allclose(loss, wl, rtol=1e-12, atol=1e-14)
    g = np.concatenate([oracle.kl_slice_bwd(x[:, o:o + w], o, lab[:, None], one, lse, coef=0.5)
                        for o, w in cuts], axis=1)
    np.testing.assert_allclose(g, wg, rtol=1e-12, atol=1e-16)


def test_kl_slice_of_minus_inf_is_left_out():
    """A slice with no finite value and no teacher entry has z = 0, a = 0
    and leaves the merge unchanged."""
    n, V, k = 3, 60, 4
    x = rows_f32(n, V)
    x[:, 20:40] = -np.inf
    ids = np.array([[0, 1, 45, 59], [2, 3, 4, 5], [41, 42, 43, 44]], dtype=np.uint32)
    p = renorm_probs(n, k)
    parts, (loss, lse) = _sliced(x, ids, p, _cuts(V, (20, 20, 20)))
    np.testing.assert_array_equal(parts[1], np.zeros((n, 4)))
    wl, wlse, _ = oracle.kl(x, ids, p, want_grad=False)
    np.testing.assert_allclose(loss, wl, rtol=1e-12)
    np.testing.assert_allclose(lse, wlse, rtol=1e-13)


def test_kl_slices_finite_differences():
    """Central differences of the merged loss in every logit equal the slice
    gradients formed from the merged lse (coef 1)."""
    h = 2.0 ** -12
    V, k = 12, 4
    x = rows_f32(1, V, 1.5)
    ids = np.array([[0, 5, 6, 11]], dtype=np.uint32)
    p = renorm_probs(1, k)
    cuts = _cuts(V, (5, 7))
    _, (_, lse) = _sliced(x, ids, p, cuts)
    g = np.concatenate([oracle.kl_slice_bwd(x[:, o:o + w], o, ids, p, lse)
                        for o, w in cuts], axis=1)
    for j in range(V):
        xp = x.copy(); xp[0, j] += np.float32(h)
        xm = x.copy(); xm[0, j] -= np.float32(h)
        lp = _sliced(xp, ids, p, cuts)[1][0][0]
        lm = _sliced(xm, ids, p, cuts)[1][0][0]
        assert abs((lp - lm) / (2 * h) - g[0, j]) < 1e-7
