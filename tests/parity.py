"""Comparison rules between the HIP path and the float64 oracle.

Loss: within 1e-5 relative (float32 logits) or 2e-3 relative (bf16), plus
an absolute floor of 1e-6 for losses near 0, where the float32 logsumexp
limits any implementation to a few 1e-7 absolute.

Gradient, float32 logits (every bound must hold):
  * each entry within 1e-6 absolute, as scaled, for a scale up to 1 (and
    1e-6 * scale above it: the scale is a plain factor);
  * each entry within 1e-3 relative (floors below), so that a zeroed,
    stale, misplaced or mis-scaled entry fails however small it is;
  * each row within 1e-5 + 4 ulp_f32(|lse|) relative L2.  Every
    p_S = exp(s - lse) carries the absolute error of the float32 logsumexp
    as a relative error, a few ulp of lse; the rest is the exponential's
    own rounding.
Gradient, bf16 logits: each entry within max(2e-3 |g_ref|, one bf16 ulp of
g_ref) -- a single round-to-nearest-even into bf16 already errs by up to
half an ulp, 2^-8 relative at worst -- and each row within 2e-3 relative L2
of the correctly rounded reference RNE_bf16(g_ref).

Floors, both dtypes:
  * at a target entry (the label, or a teacher id), g = coef (p_S - p_T) is
    formed in float32 and the two terms may cancel, so the error there is
    absolute: the float32 relative error of p_S (its exponent
    (s - max) - ln S carries a few float32 ulp at |s - lse| <= 20, the
    range where p_S can be close enough to p_T to cancel) times
    coef max(p_S, p_T).  The floor is TGT_REL * |coef| * max(p_S, p_T) with
    TGT_REL = 2^-16, at target entries only;
  * entries below 2^-100 in magnitude (float32 exponentials near
    underflow) are not held to the relative bounds.
Top-k ids bit-exact; top-k probabilities within 1e-5 relative (absolute
floor 1e-12).  Slice accumulate bit-exact.
"""
import numpy as np

LOSS_RTOL_F32 = 1e-5
LOSS_ATOL_F32 = 1e-6
GRAD_ATOL_F32 = 1e-6
GRAD_ELEM_RTOL_F32 = 1e-3
GRAD_ROW_RTOL_F32 = 1e-5
LOSS_RTOL_BF16 = 2e-3
GRAD_RTOL_BF16 = 2e-3
TGT_REL = 2.0 ** -16
TINY = 2.0 ** -100
PROB_RTOL = 1e-5
PROB_ATOL = 1e-12


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def bf16_ulp(x):
    """One unit in the last place of bf16 at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -133)))
    return np.exp2(np.maximum(e, -126.0) - 7.0)


def f32_ulp(x):
    """One unit in the last place of float32 at |x| (24 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -149)))
    return np.exp2(np.maximum(e, -126.0) - 23.0)


def check_loss(got, want, dtype, what="loss"):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if dtype == "bf16":
        tol = LOSS_RTOL_BF16 * np.abs(want) + LOSS_ATOL_F32
    else:
        tol = LOSS_RTOL_F32 * np.abs(want) + LOSS_ATOL_F32
    err = np.abs(got - want)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (
        f"{what}: {bad.size} rows out of tolerance, first row {bad[0]}: "
        f"got {got[bad[0]]!r} want {want[bad[0]]!r}")


def f64_to_bf16_rne(x):
    """float64 -> nearest bf16 value (ties to even), as float64.  The float64
    value is first rounded to float32; for the magnitudes checked here that
    intermediate rounding cannot move a value across a bf16 rounding point
    except at exact float32 ties, which a random gradient does not hit."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def dense_target(shape, ids, probs, coef):
    """coef * t as a dense float64 array: t[r, ids[r, q]] = probs[r, q] (ids
    outside [0, V) ignored).  Cross-entropy: ids = labels[:, None],
    probs = 1."""
    n, V = shape
    t = np.zeros((n, V))
    ids = np.asarray(ids).astype(np.int64).reshape(n, -1)
    p = np.broadcast_to(np.asarray(probs, dtype=np.float64), ids.shape)
    ok = (ids >= 0) & (ids < V)
    r = np.broadcast_to(np.arange(n)[:, None], ids.shape)
    np.add.at(t, (r[ok], ids[ok]), p[ok] * float(coef))
    return t


def ce_target(shape, labels, coef):
    lab = np.asarray(labels).astype(np.int64).reshape(-1, 1)
    return dense_target(shape, lab, 1.0, coef)


def _bad(what, ok, g, want, extra=""):
    bad = np.argwhere(~ok)
    assert bad.size == 0, (
        f"{what}: {len(bad)} entries out of tolerance{extra}, first {tuple(bad[0])}: "
        f"got {g[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")


def check_grad(got, want, dtype, coef=1.0, what="grad", tgt=None, lse=None):
    """got: float32 array, or uint16 bf16 bits; want: float64, the exact
    scaled gradient coef (p_S - t); coef: the gradient scale used; tgt: the
    scaled target coef t (dense, as dense_target builds it; None: no target
    entries); lse: the oracle's logsumexp per row (None: taken as 0)."""
    want = np.asarray(want, dtype=np.float64)
    t = np.zeros_like(want) if tgt is None else np.asarray(tgt, dtype=np.float64)
    assert t.shape == want.shape, (t.shape, want.shape)
    # at target entries: coef max(p_S, p_T) = max(|want + t|, |t|)
    floor = np.where(t != 0.0, TGT_REL * np.maximum(np.abs(want + t), np.abs(t)), 0.0)
    floor = np.maximum(floor, TINY)
    if dtype == "bf16":
        g = bf16_bits_to_f64(got)
        err = np.abs(g - want)
        tol = np.maximum(np.maximum(GRAD_RTOL_BF16 * np.abs(want), bf16_ulp(want)), floor)
        _bad(what, err <= tol, g, want)
        ref = f64_to_bf16_rne(want)
        num = np.sqrt(((g - ref) ** 2).sum(axis=-1))
        den = np.maximum(np.sqrt((want ** 2).sum(axis=-1)), 1e-30)
        rel = num / den
        assert (rel <= GRAD_RTOL_BF16).all(), f"{what}: row rel-L2 {rel.max():.3e}"
        return
    g = np.asarray(got, dtype=np.float64)
    err = np.abs(g - want)
    atol = GRAD_ATOL_F32 * max(1.0, abs(float(coef)))
    _bad(what, err <= atol, g, want, f" (beyond {atol} absolute)")
    _bad(what, err <= np.maximum(GRAD_ELEM_RTOL_F32 * np.abs(want), floor), g, want,
         " (element relative)")
    L = np.zeros(want.shape[:-1]) if lse is None else np.asarray(lse, dtype=np.float64)
    bound = GRAD_ROW_RTOL_F32 + 4.0 * f32_ulp(L)
    num = np.sqrt((err ** 2).sum(axis=-1))
    den = np.maximum(np.sqrt((want ** 2).sum(axis=-1)), 1e-30)
    rel = num / den
    worst = np.unravel_index(np.argmax(rel / bound), rel.shape) if rel.size else ()
    assert (rel <= bound).all(), (
        f"{what}: row rel-L2 {rel[worst]:.3e} > {np.broadcast_to(bound, rel.shape)[worst]:.3e}"
        f" at row {worst}")


def check_topk(got_ids, got_probs, want_ids, want_probs, what="topk"):
    got_ids = np.asarray(got_ids).astype(np.int64)
    want_ids = np.asarray(want_ids).astype(np.int64)
    mism = np.argwhere(got_ids != want_ids)
    assert mism.size == 0, (
        f"{what}: ids differ at {len(mism)} places, first {tuple(mism[0])}: "
        f"row got {got_ids[mism[0][0]][:8]} want {want_ids[mism[0][0]][:8]}")
    gp = np.asarray(got_probs, dtype=np.float64)
    wp = np.asarray(want_probs, dtype=np.float64)
    err = np.abs(gp - wp)
    bad = np.argwhere(~(err <= PROB_RTOL * np.abs(wp) + PROB_ATOL))
    assert bad.size == 0, (
        f"{what}: probs out of tolerance at {tuple(bad[0])}: got {gp[tuple(bad[0])]!r} "
        f"want {wp[tuple(bad[0])]!r}")
