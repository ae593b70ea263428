"""The split cross-entropy calls through the C ABI -- forward only, backward
from the saved logsumexp, mean loss on the device -- against the float64
oracle on the same seeded inputs.  Tolerances are in tests/parity.py.
Needs an MI355X."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gen import inputs as gi
from gen.inputs import to_host_bytes
from tests.parity import ce_target, check_grad, check_loss

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def vl():
    import vocab_softmax_loss_amd as m  # raises if libvl.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def dname(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def offset_rows(x):
    """The same values in a view one element past a 16-byte boundary."""
    n, V = x.shape
    base = torch.empty(n * V + 1, dtype=x.dtype, device=x.device)
    y = base[1:].view(n, V)
    y.copy_(x)
    assert y.data_ptr() % 16 != 0
    return y


def run_split(vl, x, labels, rng, scale, misalign=False):
    """Forward, then backward from the forward's lse.  Also checks that the
    forward leaves the logits untouched."""
    out = offset_rows(x) if misalign else x.clone()
    n = x.shape[0]
    before = to_host_bytes(out)
    loss = torch.full((n,), float("nan"), device=x.device)
    lse = torch.full((n,), float("nan"), device=x.device)
    vl.vl_ce_fwd(out, labels, loss, lse, rng=rng)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bytes(out), before), "the forward wrote the logits"
    lse_h = lse.cpu().numpy()
    vl.vl_ce_bwd(out, labels, lse, rng=rng, scale=scale)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse_h, to_host_bytes(out)


def assert_split(vl, x, labels, rng, scale, misalign=False):
    loss, lse, g = run_split(vl, x, labels, rng, scale, misalign)
    host = to_host_bytes(x)
    lab = labels.cpu().numpy()
    ol, olse, og = oracle.ce(host, lab, rng=rng, scale=scale)
    check_loss(loss, ol, dname(x))
    check_loss(lse, olse, dname(x), "lse")
    # the backward on its own: the oracle's backward from the same saved lse
    tgt = ce_target(og.shape, lab, scale)
    check_grad(g, oracle.ce_bwd(host, lab, lse, rng=rng, scale=scale), dname(x), scale,
               "grad from the saved lse", tgt=tgt, lse=lse)
    # end to end: the exact gradient
    check_grad(g, og, dname(x), scale, tgt=tgt, lse=olse)


def f32_ulp(x):
    return float(np.spacing(np.float32(abs(x))))


def run_mean(vl, loss_t, rng):
    mean = torch.full((1,), float("nan"), device=DEV)
    vl.vl_loss_mean(loss_t, mean, rng=rng)
    torch.cuda.synchronize()
    return float(mean.cpu().numpy()[0])


# ------------------------------------------------------------ page fixture

def test_ce_split_page_fixture(vl):
    g = json.load(open(os.path.join(GOLDEN, "ce_page_tiny.json")))
    c = gi.page_ce_tiny()
    x = torch.from_numpy(c["logits"]).to(DEV)
    lab = torch.from_numpy(c["labels"]).to(DEV)
    loss, lse, grad = run_split(vl, x, lab, c["rng"], c["scale"])
    check_loss(loss, g["loss"], "f32")
    check_loss(lse, g["lse"], "f32", "lse")
    want = np.array(g["grad"])
    check_grad(grad, want, "f32", c["scale"], tgt=ce_target(want.shape, c["labels"], c["scale"]),
               lse=np.array(g["lse"]))
    m = run_mean(vl, torch.from_numpy(loss).to(DEV), c["rng"])
    assert abs(m - g["mean_loss"]) < 1e-4  # the page's own bound
    assert abs(m - oracle.loss_mean(loss, c["rng"])) <= f32_ulp(m)


# ------------------------------------------------------------ forward + backward

CE_V = [1, 3, 8, 100, 511, 512, 1001, 2048, 2049, 4096, 8192, 8196, 32000, 32768, 32772,
        65536, 100003]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", CE_V)
def test_ce_split_shapes(vl, dtype, V):
    ntok = 9
    x = gi.normal_logits(ntok, V, 2.5, 1100 + V, DEV, TDT[dtype])
    lab = gi.uniform_labels(ntok, V, 1200 + V, DEV)
    lab[0] = 0
    lab[1] = V - 1
    rng = (4, 1, 3) if V % 2 else None
    assert_split(vl, x, lab, rng, 1.0 / 7)


# Several rows per workgroup on the persistent grid (hundreds of rows), for
# both block sizes (one wave per row up to 512 vectors, four above).
@pytest.mark.parametrize("dtype,V", [("f32", 32000), ("bf16", 30000), ("f32", 40008),
                                     ("bf16", 151936), ("f32", 2000), ("bf16", 4096)])
def test_ce_split_multirow(vl, dtype, V):
    ntok = 640 if V <= 40008 else 160
    x = gi.normal_logits(ntok, V, 3.0, 1300 + V, DEV, TDT[dtype])
    lab = gi.uniform_labels(ntok, V, 1400 + V, DEV)
    assert_split(vl, x, lab, (160, 40, 150), 1.0 / 440)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ce_split_misaligned(vl, dtype):
    x = gi.normal_logits(33, 4100, 2.0, 1500, DEV, TDT[dtype])
    lab = gi.uniform_labels(33, 4100, 1501, DEV)
    assert_split(vl, x, lab, (11, 2, 9), 0.5, misalign=True)


def test_ce_split_special_rows(vl):
    V = 4096
    x = gi.normal_logits(6, V, 2.0, 1600, DEV)
    x[0] = 1.5                       # uniform row: loss ln V
    x[1, :100] = -float("inf")       # -inf entries have zero probability
    x[2, 17] = 60.0                  # dominant label: loss ~ 0
    x[3] = -float("inf"); x[3, 5] = 0.0  # one finite entry
    x[4] *= 20.0                     # wide range
    lab = torch.tensor([3, 150, 17, 5, 9, 4095], dtype=torch.int32, device=DEV)
    assert_split(vl, x, lab, None, 0.25)


def test_ce_split_lm_small(vl):
    """The language-model recipe (boosted labels, prompt mask), 2 x 512 rows."""
    c = gi.ce_lm(DEV, seed=12, nseq=2)
    assert_split(vl, c["logits"], c["labels"], c["rng"], c["scale"])


def test_ce_split_zero_rows_and_empty_range(vl):
    z = torch.empty((0, 100), device=DEV)
    e = torch.empty(0, device=DEV)
    vl.vl_ce_fwd(z, torch.empty(0, dtype=torch.int32, device=DEV), e, e)
    vl.vl_ce_bwd(z, torch.empty(0, dtype=torch.int32, device=DEV), e)
    x = gi.normal_logits(8, 1000, 2.0, 1700, DEV)
    lab = gi.uniform_labels(8, 1000, 1701, DEV)
    loss, lse, g = run_split(vl, x, lab, (8, 3, 3), 1.0)  # empty range
    assert not loss.any() and not lse.any() and not g.any()


def test_ce_split_invalid_label(vl):
    """label >= V: NaN loss; the gradient is the softmax part alone (what
    the oracle's backward gives, whose one-hot never matches)."""
    V = 3000
    x = gi.normal_logits(4, V, 2.0, 1800, DEV)
    lab = torch.tensor([5, V, 7, 0x7FFFFFFF], dtype=torch.int32, device=DEV)
    loss, lse, g = run_split(vl, x, lab, None, 0.5)
    assert np.isnan(loss[1]) and np.isnan(loss[3])
    assert np.isfinite(loss[[0, 2]]).all() and np.isfinite(lse).all()
    host = to_host_bytes(x)
    labh = lab.cpu().numpy()
    want = oracle.ce_bwd(host, labh, lse, scale=0.5)
    check_grad(g, want, "f32", 0.5, tgt=ce_target(want.shape, labh, 0.5), lse=lse)


def test_ce_bwd_uses_the_given_lse(vl):
    """The backward takes lse as given: each row's lse raised by its own
    offset divides that row's softmax part by exp(offset)."""
    V = 5000
    x = gi.normal_logits(5, V, 2.0, 1900, DEV)
    lab = gi.uniform_labels(5, V, 1901, DEV)
    lse = torch.empty(5, device=DEV)
    vl.vl_ce_fwd(x, lab, torch.empty(5, device=DEV), lse)
    lse += torch.tensor([0.0, 1.0, 2.5, 0.125, 6.0], device=DEV)
    out = x.clone()
    vl.vl_ce_bwd(out, lab, lse, scale=2.0)
    torch.cuda.synchronize()
    labh, lseh = lab.cpu().numpy(), lse.cpu().numpy()
    want = oracle.ce_bwd(to_host_bytes(x), labh, lseh, scale=2.0)
    check_grad(to_host_bytes(out), want, "f32", 2.0, tgt=ce_target(want.shape, labh, 2.0),
               lse=lseh)


# ------------------------------------------------------------ mean loss

@pytest.mark.parametrize("n", [1, 7, 1000, 16384, 100003])
@pytest.mark.parametrize("rng", [None, (512, 128, 512), (7, 2, 5), (3, 1, 1)])
def test_loss_mean(vl, n, rng):
    g = torch.Generator(device="cpu").manual_seed(n)
    loss = (torch.rand(n, generator=g) * 10).to(DEV)
    m = run_mean(vl, loss, rng)
    want = oracle.loss_mean(loss.cpu().numpy(), rng)
    assert abs(m - want) <= f32_ulp(want), (m, want)
    assert run_mean(vl, loss, rng) == m  # same bits every run


def test_loss_mean_empty(vl):
    assert run_mean(vl, torch.empty(0, device=DEV), None) == 0.0
    assert run_mean(vl, torch.ones(6, device=DEV), (6, 2, 2)) == 0.0


def test_split_mean_matches_fused_loss(vl):
    """Forward-only loss and fused forward+backward loss over the same rows
    give the same mean within float32 rounding."""
    c = gi.ce_lm(DEV, seed=13, nseq=2)
    x, lab, rng = c["logits"], c["labels"], c["rng"]
    n = x.shape[0]
    l1 = torch.empty(n, device=DEV)
    l2 = torch.empty(n, device=DEV)
    vl.vl_ce_fwd(x, lab, l1, rng=rng)
    vl.vl_ce_fwd_bwd(x.clone(), lab, l2, rng=rng, scale=c["scale"])
    torch.cuda.synchronize()
    m1, m2 = run_mean(vl, l1, rng), run_mean(vl, l2, rng)
    assert abs(m1 - m2) <= 1e-5 * abs(m2)
