"""The vocabulary-slice KL calls through the C ABI -- per-slice statistics,
their merge, and the slice gradient from the merged lse -- against the
float64 oracle on the same seeded inputs: the parts against the oracle's
parts, and the merged loss, lse and gradient against the oracle's
whole-row KL.  Tolerances are in tests/parity.py.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
from gen import inputs as gi
from gen.inputs import to_host_bytes
from tests.parity import bf16_bits_to_f64, ce_target, check_grad, check_loss, dense_target

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def vl():
    import vocab_softmax_loss_amd as m  # raises if libvl.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def dname(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def cuts_of(V, widths):
    offs = np.cumsum([0] + list(widths))
    assert offs[-1] == V
    return [(int(o), int(w)) for o, w in zip(offs[:-1], widths)]


def widen(h):
    return bf16_bits_to_f64(h) if h.dtype == np.uint16 else h.astype(np.float64)


def run_sliced(vl, x, ids, probs, cuts, rng, coef, layout):
    """The three calls over the slices of x.  layout "window": each slice is
    a column window of one copy of x (row stride V); "dense": each slice is
    its own contiguous [ntok][width] tensor; "misaligned": dense, one
    element past a 16-byte boundary.  Returns (parts, loss, lse, gradient
    rows as host bytes)."""
    n, V = x.shape
    parts = torch.full((len(cuts), n, 4), float("nan"), device=DEV)
    if layout == "window":
        buf = x.clone()
        slices = [buf[:, o:o + w] for o, w in cuts]
    else:
        slices = []
        for o, w in cuts:
            if layout == "misaligned":
                base = torch.empty(n * w + 1, dtype=x.dtype, device=DEV)
                s = base[1:].view(n, w)
                assert s.data_ptr() % 16 != 0
            else:
                s = torch.empty((n, w), dtype=x.dtype, device=DEV)
            s.copy_(x[:, o:o + w])
            slices.append(s)
    for i, (o, w) in enumerate(cuts):
        vl.vl_kl_slice_fwd(slices[i], o, ids, probs, parts[i], rng=rng)
    loss = torch.full((n,), float("nan"), device=DEV)
    lse = torch.full((n,), float("nan"), device=DEV)
    vl.vl_kl_slice_merge(parts, loss, lse, rng=rng)
    for i, (o, w) in enumerate(cuts):
        vl.vl_kl_slice_bwd(slices[i], o, ids, probs, lse, rng=rng, coef=coef)
    torch.cuda.synchronize()
    g = np.concatenate([to_host_bytes(s.contiguous()) for s in slices], axis=1)
    return parts.cpu().numpy(), loss.cpu().numpy(), lse.cpu().numpy(), g


def check_parts(got, host, ids, probs, cuts, rng):
    """a exact (a maximum of the given values); z within 1e-5 relative; P
    and w within 1e-5 of the magnitudes they sum (float32 sums of k terms)."""
    idv = ids.astype(np.int64)
    for i, (o, w) in enumerate(cuts):
        want = oracle.kl_slice_part(host[:, o:o + w], o, ids, probs, rng=rng)
        g = got[i].astype(np.float64)
        assert np.array_equal(g[:, 0], want[:, 0]), f"slice {i}: anchors differ"
        assert np.all(np.abs(g[:, 1] - want[:, 1]) <= 1e-5 * want[:, 1]), f"slice {i}: z"
        s = widen(host[:, o:o + w])
        mag = np.zeros(len(want))
        for t in range(len(want)):
            j = idv[t] - o
            m = (j >= 0) & (j < w) & (probs[t] > 0)
            if m.any():
                p = probs[t][m].astype(np.float64)
                mag[t] = (p * (np.abs(np.log(p)) + np.abs(s[t, j[m]] - want[t, 0]))).sum()
        assert np.all(np.abs(g[:, 2] - want[:, 2]) <= 1e-6 * np.maximum(want[:, 2], 1)), \
            f"slice {i}: P"
        assert np.all(np.abs(g[:, 3] - want[:, 3]) <= 1e-5 * mag + 1e-6), f"slice {i}: w"


def assert_sliced(vl, x, ids, probs, cuts, rng, coef, layout="window"):
    parts, loss, lse, g = run_sliced(vl, x, ids, probs, cuts, rng, coef, layout)
    host = to_host_bytes(x)
    idh = ids.cpu().numpy().view(np.uint32)
    ph = probs.cpu().numpy()
    check_parts(parts, host, idh, ph, cuts, rng)
    ol, olse, og = oracle.kl(host, idh, ph, rng=rng, coef=coef)
    check_loss(loss, ol, dname(x))
    check_loss(lse, olse, dname(x), "lse")
    # each slice's gradient on its own, from the same lse the GPU used
    gb = np.concatenate([oracle.kl_slice_bwd(host[:, o:o + w], o, idh, ph, lse, coef=coef,
                                             rng=rng) for o, w in cuts], axis=1)
    tgt = dense_target(og.shape, idh, ph, coef)
    check_grad(g, gb, dname(x), coef, "slice gradient from the merged lse", tgt=tgt, lse=lse)
    # end to end: the whole row's exact gradient
    check_grad(g, og, dname(x), coef, tgt=tgt, lse=olse)


CASES = [
    # (dtype, ntok, V, widths, k)
    ("f32", 7, 1000, (1000,), 16),
    ("f32", 9, 4096, (2048, 2048), 64),
    ("bf16", 9, 4096, (2048, 2048), 64),
    ("f32", 5, 10007, (3333, 3337, 3337), 100),
    ("bf16", 5, 10000, (8, 9984, 8), 40),
    ("f32", 6, 32000, (16000, 16000), 64),
    ("bf16", 4, 151936, (75968, 75968), 256),
    ("f32", 3, 128256, (64128, 64128), 128),
    ("f32", 4, 640, (64,) * 10, 200),       # ten slices, 64 columns each
    ("bf16", 3, 2000, (1, 1999), 7),        # one-column slice
    ("f32", 4, 3000, (1000, 2000), 700),    # several 256-id loads per wave
    ("bf16", 4, 24576, (8192, 16384), 1030),
]


@pytest.mark.parametrize("layout", ["window", "dense"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[2]}-{len(c[3])}x")
def test_slices_match_whole_row(vl, case, layout):
    dtype, n, V, widths, k = case
    x = gi.normal_logits(n, V, 2.0, 3100 + V, DEV, TDT[dtype])
    ids = gi.distinct_ids(n, V, k, 3200 + V, DEV)
    probs = gi.softmax_probs(n, k, 1.5, 3300 + V, DEV)
    rng = (3, 1, 3) if n > 3 else None
    assert_sliced(vl, x, ids, probs, cuts_of(V, widths), rng, 1.0 / n, layout)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_slices_misaligned(vl, dtype):
    V = 4100
    x = gi.normal_logits(11, V, 2.0, 3400, DEV, TDT[dtype])
    ids = gi.distinct_ids(11, V, 33, 3401, DEV)
    probs = gi.softmax_probs(11, 33, 1.5, 3402, DEV)
    assert_sliced(vl, x, ids, probs, cuts_of(V, (1025, 3075)), (11, 2, 9), 0.5, "misaligned")


def test_slices_multirow(vl):
    """Hundreds of rows per slice: several rows per workgroup of the part
    pass's persistent grid, for both block sizes."""
    for dtype, V, widths in (("f32", 32000, (30000, 2000)), ("bf16", 12288, (4096, 8192))):
        n = 700
        x = gi.normal_logits(n, V, 3.0, 3500 + V, DEV, TDT[dtype])
        ids = gi.distinct_ids(n, V, 64, 3501 + V, DEV)
        probs = gi.softmax_probs(n, 64, 1.5, 3502 + V, DEV)
        assert_sliced(vl, x, ids, probs, cuts_of(V, widths), (350, 50, 340), 1.0 / 580)


def test_slices_every_id_in_one_chunk(vl):
    """k = V: every element of the row is a teacher entry, so every lane of
    the gradient pass takes hits from several id loads."""
    V = 512
    x = gi.normal_logits(4, V, 2.0, 3600, DEV)
    ids = gi.distinct_ids(4, V, V, 3601, DEV)
    probs = gi.softmax_probs(4, V, 1.5, 3602, DEV)
    assert_sliced(vl, x, ids, probs, cuts_of(V, (256, 256)), None, 0.25)


def test_slices_special_rows(vl):
    """-inf entries, a slice with no finite value and no teacher entry, a
    uniform row, a wide range."""
    V, k = 3000, 6
    x = gi.normal_logits(5, V, 2.0, 3700, DEV)
    x[0] = 1.5
    x[1, 1000:2000] = -float("inf")
    x[2, :10] = -float("inf")
    x[3] *= 20.0
    ids = torch.tensor([[0, 1, 2, 2999, 1500, 700],
                        [0, 1, 2, 2999, 2500, 700],
                        [10, 11, 12, 13, 14, 2000],
                        [5, 6, 7, 8, 9, 10],
                        [100, 1100, 2100, 2200, 2300, 2400]], dtype=torch.int32, device=DEV)
    probs = gi.softmax_probs(5, k, 1.5, 3701, DEV)
    assert_sliced(vl, x, ids, probs, cuts_of(V, (1000, 1000, 1000)), None, 0.5)


def test_slices_nan_logit(vl):
    """A NaN logit in one slice of a row makes that row's lse and loss NaN
    (its slice's sum is NaN and the merge keeps it); the other rows come
    out exactly as without it."""
    V, k, n = 3000, 6, 4
    x = gi.normal_logits(n, V, 2.0, 3750, DEV)
    ids = gi.distinct_ids(n, V, k, 3751, DEV)
    probs = gi.softmax_probs(n, k, 1.5, 3752, DEV)
    cuts = cuts_of(V, (1000, 1000, 1000))
    _, l0, s0, g0 = run_sliced(vl, x, ids, probs, cuts, None, 0.5, "window")
    y = x.clone()
    y[1, 2345] = float("nan")
    _, l1, s1, g1 = run_sliced(vl, y, ids, probs, cuts, None, 0.5, "window")
    assert np.isnan(l1[1]) and np.isnan(s1[1])
    keep = [0, 2, 3]
    assert np.array_equal(l1[keep], l0[keep]) and np.array_equal(s1[keep], s0[keep])
    assert np.array_equal(g1[keep], g0[keep])


def test_slices_unit_target_is_the_cross_entropy(vl):
    """k = 1, probs = 1: the merged loss and the slice gradients are the
    fused cross-entropy's."""
    V = 32000
    x = gi.normal_logits(16, V, 3.0, 3800, DEV)
    lab = gi.uniform_labels(16, V, 3801, DEV)
    one = torch.ones((16, 1), device=DEV)
    cuts = cuts_of(V, (12000, 20000))
    _, loss, _, g = run_sliced(vl, x, lab[:, None].contiguous(), one, cuts, (8, 2, 8), 1.0 / 12,
                               "window")
    host = to_host_bytes(x)
    labh = lab.cpu().numpy()
    ol, olse, og = oracle.ce(host, labh, rng=(8, 2, 8), scale=1.0 / 12)
    check_loss(loss, ol, "f32")
    check_grad(g, og, "f32", 1.0 / 12, tgt=ce_target(og.shape, labh, 1.0 / 12), lse=olse)


def test_slices_zero_rows_and_empty_range(vl):
    z = torch.empty((0, 64), device=DEV)
    e = torch.empty((0, 4), device=DEV)
    i0 = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    p0 = torch.empty((0, 2), device=DEV)
    vl.vl_kl_slice_fwd(z, 0, i0, p0, e)
    vl.vl_kl_slice_merge(torch.empty((2, 0, 4), device=DEV), torch.empty(0, device=DEV))
    vl.vl_kl_slice_bwd(z, 0, i0, p0, torch.empty(0, device=DEV))
    V = 1000
    x = gi.normal_logits(6, V, 2.0, 3900, DEV)
    ids = gi.distinct_ids(6, V, 8, 3901, DEV)
    probs = gi.softmax_probs(6, 8, 1.5, 3902, DEV)
    parts, loss, lse, g = run_sliced(vl, x, ids, probs, cuts_of(V, (500, 500)), (6, 2, 2), 1.0,
                                     "dense")
    assert not parts.any() and not loss.any() and not lse.any() and not g.any()


@pytest.mark.slow
def test_slices_bf16_151936_full(vl):
    """The large bf16 workload as two vocabulary slices of 75968, each its
    own [16384][75968] buffer, teacher top-k (k=256) by the GPU: sampled
    rows against the oracle's whole-row KL, every row's loss against the
    fused KL call, and every gradient row's sum."""
    c = gi.kl_bf16_sliced(DEV)
    x, t, k, coef = c["logits"], c["teacher"], c["k"], c["coef"]
    ntok, V = x.shape
    ids = torch.empty((ntok, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((ntok, k), device=DEV)
    vl.vl_topk_renorm(t, k, ids, probs)
    cuts = cuts_of(V, (75968, 75968))
    rows = np.unique(np.concatenate([np.random.default_rng(61).choice(ntok, 24, replace=False),
                                     [0, ntok - 1]]))
    rows_t = torch.from_numpy(rows).to(DEV)
    xh = to_host_bytes(x[rows_t])
    slices = [x[:, o:o + w].contiguous() for o, w in cuts]
    parts = torch.empty((2, ntok, 4), device=DEV)
    for i, (o, w) in enumerate(cuts):
        vl.vl_kl_slice_fwd(slices[i], o, ids, probs, parts[i])
    loss = torch.empty(ntok, device=DEV)
    lse = torch.empty(ntok, device=DEV)
    vl.vl_kl_slice_merge(parts, loss, lse)
    for i, (o, w) in enumerate(cuts):
        vl.vl_kl_slice_bwd(slices[i], o, ids, probs, lse, coef=coef)
    fused = torch.empty(ntok, device=DEV)
    vl.vl_kl_fwd_bwd(x, ids, probs, fused, coef=coef)
    torch.cuda.synchronize()
    idh = ids[rows_t].cpu().numpy().view(np.uint32)
    ph = probs[rows_t].cpu().numpy()
    ol, olse, og = oracle.kl(xh, idh, ph, coef=coef)
    check_loss(loss.cpu().numpy()[rows], ol, "bf16")
    check_loss(lse.cpu().numpy()[rows], olse, "bf16", "lse")
    g = np.concatenate([to_host_bytes(s[rows_t]) for s in slices], axis=1)
    check_grad(g, og, "bf16", coef, tgt=dense_target(og.shape, idh, ph, coef), lse=olse)
    lf, ls = fused.double(), loss.double()
    assert float(((ls - lf).abs() / lf.abs()).max()) < 1e-5
    gs = sum(s.sum(dim=1, dtype=torch.float64) for s in slices)
    want = coef * (1.0 - probs.sum(dim=1, dtype=torch.float64))
    assert float((gs - want).abs().max()) < 1e-3
