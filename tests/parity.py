"""Comparison rules between the HIP path and the float64 oracle.

Tolerances (float32 logits): per-token loss within 1e-5 relative (plus an
absolute floor of 1e-6 for losses that are themselves near 0, where the
float32 logsumexp limits any implementation to a few 1e-7 absolute); scaled
gradient entries within 1e-6 absolute for a gradient scale up to 1, and
1e-6 * scale above it (the scale is a plain factor, so the bound scales with
it).  bf16 logits: loss within 2e-3 relative; each gradient entry within
max(2e-3 |g_ref|, one bf16 ulp of g_ref, the float32 bound above) -- a
single round-to-nearest-even into bf16 already errs by up to half an ulp,
2^-8 relative at worst, and a teacher entry coef (p_S - p_T) is formed in
float32 before it is rounded, so where p_S and p_T nearly cancel it carries
the float32 absolute error of coef p_T, not a relative one -- and
every row within 2e-3 relative L2 of the correctly rounded reference
RNE_bf16(g_ref), so the bound measures the kernel's own error, not the
rounding every bf16 result carries.
Top-k ids bit-exact; top-k probabilities within 1e-5 relative (absolute
floor 1e-12).  Slice accumulate bit-exact.
"""
import numpy as np

LOSS_RTOL_F32 = 1e-5
LOSS_ATOL_F32 = 1e-6
GRAD_ATOL_F32 = 1e-6
LOSS_RTOL_BF16 = 2e-3
GRAD_RTOL_BF16 = 2e-3
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


def check_grad(got, want, dtype, coef=1.0, what="grad"):
    """got: float32 array, or uint16 bf16 bits; want: float64 (the exact
    scaled gradient); coef: the gradient scale used."""
    want = np.asarray(want, dtype=np.float64)
    if dtype == "bf16":
        g = bf16_bits_to_f64(got)
        err = np.abs(g - want)
        tol = np.maximum(np.maximum(GRAD_RTOL_BF16 * np.abs(want), bf16_ulp(want)),
                         GRAD_ATOL_F32 * max(1.0, abs(float(coef))))
        bad = np.argwhere(~(err <= tol))
        assert bad.size == 0, (
            f"{what}: {len(bad)} entries out of tolerance, first {tuple(bad[0])}: "
            f"got {g[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")
        ref = f64_to_bf16_rne(want)
        num = np.sqrt(((g - ref) ** 2).sum(axis=-1))
        den = np.maximum(np.sqrt((want ** 2).sum(axis=-1)), 1e-30)
        rel = num / den
        assert (rel <= GRAD_RTOL_BF16).all(), f"{what}: row rel-L2 {rel.max():.3e}"
        return
    g = np.asarray(got, dtype=np.float64)
    err = np.abs(g - want)
    atol = GRAD_ATOL_F32 * max(1.0, abs(float(coef)))
    bad = np.argwhere(~(err <= atol))
    assert bad.size == 0, (
        f"{what}: {len(bad)} entries beyond {atol}, first {tuple(bad[0])}: "
        f"got {g[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")


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
