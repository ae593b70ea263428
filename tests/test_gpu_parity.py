"""HIP path (through the C ABI) against the float64 oracle on the same seeded
inputs.  Tolerances are in tests/parity.py.  Needs an MI355X."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gen import inputs as gi
from gen.inputs import to_host_bytes
from tests.parity import (bf16_bits_to_f64, ce_target, check_grad, check_loss, check_topk,
                          dense_target)

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
    """The same values in a row-major view whose base is one element past a
    16-byte boundary: the 16-byte vector path cannot be used."""
    n, V = x.shape
    base = torch.empty(n * V + 1, dtype=x.dtype, device=x.device)
    y = base[1:].view(n, V)
    y.copy_(x)
    assert y.data_ptr() % 16 != 0
    return y


def run_ce(vl, x, labels, rng, scale, misalign=False):
    out = offset_rows(x) if misalign else x.clone()
    n = x.shape[0]
    loss = torch.full((n,), float("nan"), device=x.device)
    lse = torch.full((n,), float("nan"), device=x.device)
    vl.vl_ce_fwd_bwd(out, labels, loss, lse, rng=rng, scale=scale)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy(), to_host_bytes(out)


def run_kl(vl, x, ids, probs, rng, coef, misalign=False):
    out = offset_rows(x) if misalign else x.clone()
    n = x.shape[0]
    loss = torch.full((n,), float("nan"), device=x.device)
    lse = torch.full((n,), float("nan"), device=x.device)
    vl.vl_kl_fwd_bwd(out, ids, probs, loss, lse, rng=rng, coef=coef)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy(), to_host_bytes(out)


def run_topk(vl, x, k):
    n = x.shape[0]
    ids = torch.full((n, k), -1, dtype=torch.int32, device=x.device)
    probs = torch.full((n, k), float("nan"), device=x.device)
    vl.vl_topk_renorm(x, k, ids, probs)
    torch.cuda.synchronize()
    return ids.cpu().numpy().view(np.uint32), probs.cpu().numpy()


def assert_ce(vl, x, labels, rng, scale, misalign=False):
    loss, lse, g = run_ce(vl, x, labels, rng, scale, misalign)
    lab = labels.cpu().numpy()
    ol, olse, og = oracle.ce(to_host_bytes(x), lab, rng=rng, scale=scale)
    check_loss(loss, ol, dname(x))
    check_loss(lse, olse, dname(x), "lse")
    check_grad(g, og, dname(x), scale, tgt=ce_target(og.shape, lab, scale), lse=olse)


def assert_kl(vl, x, ids, probs, rng, coef, misalign=False):
    loss, lse, g = run_kl(vl, x, ids, probs, rng, coef, misalign)
    idh, ph = ids.cpu().numpy(), probs.cpu().numpy()
    ol, olse, og = oracle.kl(to_host_bytes(x), idh, ph, rng=rng, coef=coef)
    check_loss(loss, ol, dname(x))
    check_loss(lse, olse, dname(x), "lse")
    check_grad(g, og, dname(x), coef, tgt=dense_target(og.shape, idh, ph, coef), lse=olse)


# ------------------------------------------------------------ page fixtures

def test_ce_page_fixture(vl):
    g = json.load(open(os.path.join(GOLDEN, "ce_page_tiny.json")))
    c = gi.page_ce_tiny()
    x = torch.from_numpy(c["logits"]).to(DEV)
    lab = torch.from_numpy(c["labels"]).to(DEV)
    loss, lse, grad = run_ce(vl, x, lab, c["rng"], c["scale"])
    check_loss(loss, g["loss"], "f32")
    check_loss(lse, g["lse"], "f32", "lse")
    want = np.array(g["grad"])
    check_grad(grad, want, "f32", c["scale"], tgt=ce_target(want.shape, c["labels"], c["scale"]),
               lse=np.array(g["lse"]))
    assert abs(loss.sum() / 4 - g["mean_loss"]) < 1e-4  # the page's own bound


def test_kl_page_fixture(vl):
    g = json.load(open(os.path.join(GOLDEN, "kl_page_tiny.json")))
    c = gi.page_kl_tiny()
    x = torch.from_numpy(c["logits"]).to(DEV)
    ids = torch.from_numpy(c["ids"]).to(DEV)
    probs = torch.from_numpy(c["probs"]).to(DEV)
    loss, lse, grad = run_kl(vl, x, ids, probs, None, c["coef"])
    check_loss(loss, g["loss"], "f32")
    check_loss(lse, g["lse"], "f32", "lse")
    tgt = dense_target(grad.shape, c["ids"], c["probs"], c["coef"])
    for s in g["grad_samples"]:
        r, cols = s["row"], s["cols"]
        check_grad(grad[r, cols], np.array(s["grad"]), "f32", c["coef"], tgt=tgt[r, cols],
                   lse=g["lse"][r])
    # the page's own metric: relative L2 of the loss vector below 1e-4
    want = np.array(g["loss"])
    assert np.linalg.norm(loss - want) / np.linalg.norm(want) < 1e-4


# ------------------------------------------------------------ CE

def test_ce_tiny_config(vl):
    c = gi.ce_tiny(DEV)
    assert_ce(vl, c["logits"], c["labels"], c["rng"], c["scale"])


CE_V = [1, 3, 8, 100, 511, 512, 1001, 2048, 2049, 4096, 8192, 8196, 16384, 16388, 32000,
        32768, 32772, 65536, 65544, 100003, 155648, 155656]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", CE_V)
def test_ce_shapes(vl, dtype, V):
    ntok = 9
    x = gi.normal_logits(ntok, V, 2.5, 100 + V, DEV, TDT[dtype])
    lab = gi.uniform_labels(ntok, V, 200 + V, DEV)
    lab[0] = 0
    lab[1] = V - 1
    rng = (4, 1, 3) if V % 2 else None
    assert_ce(vl, x, lab, rng, 1.0 / 7)


def test_ce_zero_rows_and_single_row(vl):
    x = torch.empty((0, 100), device=DEV)
    vl.vl_ce_fwd_bwd(x, torch.empty(0, dtype=torch.int32, device=DEV),
                     torch.empty(0, device=DEV))
    c = gi.ce_tiny(DEV, ntok=1, V=32000)
    assert_ce(vl, c["logits"], c["labels"], None, 1.0)


def test_ce_special_rows(vl):
    V = 4096
    x = gi.normal_logits(6, V, 2.0, 7, DEV)
    x[0] = 1.5                       # uniform row: loss ln V
    x[1, :100] = -float("inf")       # -inf entries have zero probability
    x[2, 17] = 60.0                  # dominant label: loss ~ 0
    x[3] = -float("inf"); x[3, 5] = 0.0  # one finite entry
    x[4] *= 20.0                     # wide range
    lab = torch.tensor([3, 150, 17, 5, 9, 4095], dtype=torch.int32, device=DEV)
    assert_ce(vl, x, lab, None, 0.25)


def test_ce_loss_range_all_out(vl):
    x = gi.normal_logits(8, 1000, 2.0, 9, DEV)
    lab = gi.uniform_labels(8, 1000, 10, DEV)
    loss, lse, g = run_ce(vl, x, lab, (8, 3, 3), 1.0)  # empty range
    assert not loss.any() and not lse.any() and not g.any()


def test_ce_lm_small(vl):
    """The LM-shaped recipe (boosted labels, prompt mask) at 2 x 512 rows."""
    c = gi.ce_lm(DEV, nseq=2)
    assert_ce(vl, c["logits"], c["labels"], c["rng"], c["scale"])


# Several rows per workgroup: the persistent grid has at most a few blocks
# per CU, so 600+ rows give every block a sequence of rows, which exercises
# the next-row pipelines (LDS prefetch, register refill) and the row-parity
# LDS buffers.  V picks the variant: 32000 float32 and 30000 bf16 are staged
# with an LDS prefetch, 40008 float32 is online, 40008 bf16 refills
# registers, 8000 bf16 runs two blocks per CU.
MULTIROW = [("f32", 32000), ("bf16", 30000), ("f32", 40008), ("bf16", 40008), ("bf16", 8000)]


@pytest.mark.parametrize("dtype,V", MULTIROW)
def test_ce_multirow(vl, dtype, V):
    ntok = 640
    x = gi.normal_logits(ntok, V, 3.0, 600 + V, DEV, TDT[dtype])
    lab = gi.uniform_labels(ntok, V, 700 + V, DEV)
    assert_ce(vl, x, lab, (160, 40, 150), 1.0 / 440)


@pytest.mark.parametrize("dtype,V", MULTIROW)
def test_kl_multirow(vl, dtype, V):
    ntok, k = 640, 96
    x = gi.normal_logits(ntok, V, 2.0, 800 + V, DEV, TDT[dtype])
    ids = gi.distinct_ids(ntok, V, k, 900 + V, DEV)
    probs = gi.softmax_probs(ntok, k, 1.5, 1000 + V, DEV)
    assert_kl(vl, x, ids, probs, None, 1024.0 / ntok)


# Every row-kernel variant with several rows per workgroup, with a loss
# range: ntok is three times the largest grid the variant can launch plus
# one (256 CUs x the most blocks of its size a CU can hold: 32 of 64
# threads, 8 of 256, 4 of 512, 2 of 1024), so every workgroup walks at
# least three in-range rows (the row-parity LDS slots and bitmaps, the
# one-row-late bitmap clear, the next row's target fetch, and the LDS
# prefetch or register refill where the variant has one) and then
# write-only rows.  (dtype, V, threads per block) in launch-table order;
# the last two float32 / bf16 entries are the online and register-refill
# variants, and "unaligned" rows take the element path.
VARIANTS = [
    ("f32", 200, 64), ("f32", 500, 64), ("f32", 1000, 64), ("f32", 2000, 64),
    ("f32", 4000, 256), ("f32", 8000, 256), ("f32", 16000, 512), ("f32", 32000, 1024),
    ("f32", 40008, 1024),
    ("bf16", 504, 64), ("bf16", 1000, 64), ("bf16", 2000, 64), ("bf16", 8000, 256),
    ("bf16", 32000, 512), ("bf16", 40008, 1024), ("bf16", 160000, 1024),
    ("unaligned-f32", 4096, 256), ("unaligned-bf16", 4096, 256),
]


def _variant_rows(threads):
    return 3 * 256 * (2048 // threads) + 1


def _check_chunked(kind, host, got, loss, lse, tg, probs, rng, coef, dtype):
    """Every row against the oracle, in chunks of about 2^25 values."""
    n, V = host.shape
    step = max(1, (1 << 25) // V)
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        ri = np.arange(r0, r1)
        if kind == "ce":
            ol, olse, og = oracle.ce(host[r0:r1], tg[r0:r1], rng=rng, scale=coef, row_index=ri)
            tgt = ce_target(og.shape, tg[r0:r1], coef)
        else:
            ol, olse, og = oracle.kl(host[r0:r1], tg[r0:r1], probs[r0:r1], rng=rng, coef=coef,
                                     row_index=ri)
            tgt = dense_target(og.shape, tg[r0:r1], probs[r0:r1], coef)
        check_loss(loss[r0:r1], ol, dtype, f"loss rows {r0}-{r1}")
        check_loss(lse[r0:r1], olse, dtype, f"lse rows {r0}-{r1}")
        check_grad(got[r0:r1], og, dtype, coef, f"grad rows {r0}-{r1}", tgt=tgt, lse=olse)


@pytest.mark.parametrize("kind", ["ce", "kl"])
@pytest.mark.parametrize("dtype,V,threads", VARIANTS)
def test_variant_multirow_with_range(vl, kind, dtype, V, threads):
    mis = dtype.startswith("unaligned")
    dt = dtype.split("-")[-1]
    ntok = _variant_rows(threads)
    print(f"variant {dtype} V={V} threads={threads} ntok={ntok} {kind}", flush=True)
    x = gi.normal_logits(ntok, V, 2.5, 4000 + V + threads, DEV, TDT[dt])
    rng = (7, 1, 6)
    coef = 1.0 / 300
    if kind == "ce":
        tg = gi.uniform_labels(ntok, V, 4100 + V, DEV)
        loss, lse, g = run_ce(vl, x, tg, rng, coef, misalign=mis)
        probs = None
    else:
        k = min(V, 48)
        tg = gi.distinct_ids(ntok, V, k, 4200 + V, DEV)
        pt = gi.softmax_probs(ntok, k, 1.5, 4300 + V, DEV)
        loss, lse, g = run_kl(vl, x, tg, pt, rng, coef, misalign=mis)
        probs = pt.cpu().numpy()
    _check_chunked(kind, to_host_bytes(x), g, loss, lse, tg.cpu().numpy(), probs, rng, coef,
                   dt)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [4096, 32000, 40008])
def test_kl_padded_teacher_list(vl, dtype, V):
    """A teacher list padded with repeated ids at probability 0 (the
    zero-probability entries take no part): the same result as the
    oracle, which sums the probabilities of repeated ids.  The padding
    repeats the row's first id, or an id alone in its 16-byte vector."""
    ntok, k, kreal = 40, 24, 15
    x = gi.normal_logits(ntok, V, 2.0, 4400 + V, DEV, TDT[dtype])
    ids = gi.distinct_ids(ntok, V, k, 4500 + V, DEV)
    probs = gi.softmax_probs(ntok, k, 1.5, 4600 + V, DEV)
    probs[:, kreal:] = 0.0
    probs[:, :kreal] /= probs[:, :kreal].sum(dim=1, keepdim=True)
    ids[:, kreal:] = ids[:, :1]            # repeats of the first (real) id
    ids[1::2, kreal + 2:] = ids[1::2, 3:4]  # and of another on odd rows
    assert_kl(vl, x, ids, probs, None, 1.0 / 40)


# ------------------------------------------------------------ KL

# (20000, 1500): more teacher ids than threads in the 1024-thread float32
# block with the LDS prefetch, so threads handle several ids each.  Either
# side of each variant boundary: float32 16384 | 16388 (512 x 8 | 1024 x 8
# with the LDS prefetch), 32768 | 32772 (staged | online); bf16 155648 |
# 155656 (register refill | online).
KL_VK = [(1, 1), (8, 3), (512, 16), (1001, 64), (2049, 5), (8192, 128), (16384, 64),
         (16388, 64), (32000, 64), (20000, 1500), (32768, 100), (32772, 200), (65544, 256),
         (131072, 2048), (151936, 256), (155648, 64), (155656, 64),
         (1 << 19, 64)]  # the largest KL vocabulary: two 64 KB bitmaps in LDS


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [4096, 32000, 40008])
def test_kl_clustered_ids(vl, dtype, V):
    """Teacher ids packed into few 16-byte vectors (1 to 8 targets per
    vector), beside vectors holding a single one: both ways of writing the
    target entries, in the staged, prefetched, online and register-refill
    variants."""
    ntok, k = 300, 40
    g = torch.Generator()
    g.manual_seed(V)
    rows = []
    for r in range(ntok):
        base = torch.randperm(V // 8, generator=g)[:26] * 8
        single = base[4:] + (r + torch.arange(22)) % 8  # one target in each
        rows.append(torch.cat([base[0] + torch.arange(8), base[1] + torch.arange(5),
                               base[2] + torch.tensor([0, 7]),
                               base[3] + torch.tensor([2, 3, 4]), single]))
    ids = torch.stack([x[torch.randperm(k, generator=g)] for x in rows]).to(torch.int32)
    assert ids.shape == (ntok, k) and all(torch.unique(x).numel() == k for x in ids)
    ids = ids.to(DEV)
    x = gi.normal_logits(ntok, V, 2.0, 1100 + V, DEV, TDT[dtype])
    probs = gi.softmax_probs(ntok, k, 1.5, 1200 + V, DEV)
    assert_kl(vl, x, ids, probs, None, 1024.0 / ntok)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,k", KL_VK)
def test_kl_shapes(vl, dtype, V, k):
    ntok = 6
    x = gi.normal_logits(ntok, V, 2.0, 300 + V, DEV, TDT[dtype])
    ids = gi.distinct_ids(ntok, V, k, 400 + V, DEV)
    probs = gi.softmax_probs(ntok, k, 1.5, 500 + V, DEV)
    rng = (3, 0, 2) if V % 2 else None
    assert_kl(vl, x, ids, probs, rng, 1024.0 / ntok)


def test_kl_zero_probs_and_unnormalised(vl):
    V, k, ntok = 3000, 32, 5
    x = gi.normal_logits(ntok, V, 2.0, 11, DEV)
    ids = gi.distinct_ids(ntok, V, k, 12, DEV)
    probs = gi.softmax_probs(ntok, k, 1.0, 13, DEV)
    probs[:, ::3] = 0.0   # zero-probability entries: no loss term
    probs[1] *= 0.5       # used as given, no renormalisation
    assert_kl(vl, x, ids, probs, None, 0.5)


def test_kl_large_small_rows(vl):
    c = gi.kl_large(DEV, ntok=8, V=128256, k=128)
    assert_kl(vl, c["logits"], c["ids"], c["probs"], None, c["coef"])


def test_kl_invalid_id_gives_nan_loss_only(vl):
    V, k = 1000, 4
    x = gi.normal_logits(3, V, 2.0, 21, DEV)
    ids = torch.tensor([[1, 2, 3, 4], [5, 6, 7, 5000], [8, 9, 10, 11]], dtype=torch.int32,
                       device=DEV)
    probs = torch.full((3, k), 0.25, device=DEV)
    loss, _, g = run_kl(vl, x, ids, probs, None, 1.0)
    assert np.isnan(loss[1]) and np.isfinite(loss[[0, 2]]).all()
    idh, ph = ids.cpu().numpy()[[0, 2]], probs.cpu().numpy()[[0, 2]]
    ol, olse, og = oracle.kl(to_host_bytes(x)[[0, 2]], idh, ph, coef=1.0)
    check_loss(loss[[0, 2]], ol, "f32")
    check_grad(g[[0, 2]], og, "f32", 1.0, tgt=dense_target(og.shape, idh, ph, 1.0), lse=olse)


# ------------------------------------------------------------ top-k

def topk_rows(kind, ntok, V, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    if kind == "normal":
        x = torch.randn((ntok, V), generator=g, device=DEV) * 2.0
    elif kind == "ties":
        x = torch.randint(-4, 5, (ntok, V), generator=g, device=DEV).float() * 0.5
    elif kind == "ascending":
        x = torch.arange(V, device=DEV, dtype=torch.float32).repeat(ntok, 1) * 1e-3
    elif kind == "descending":
        x = -torch.arange(V, device=DEV, dtype=torch.float32).repeat(ntok, 1) * 1e-3
    elif kind == "zeros":  # -0 and +0 mixed, a few positives
        x = torch.zeros((ntok, V), device=DEV)
        x[:, 1::2] = -0.0
        x[:, 7::97] = 1.0
    elif kind == "neg_inf":
        x = torch.full((ntok, V), -float("inf"), device=DEV)
        x[:, 3::11] = torch.randn((ntok, len(range(3, V, 11))), generator=g, device=DEV)
    elif kind == "stride":  # every large value in one lane's stride class
        x = torch.randn((ntok, V), generator=g, device=DEV) - 10.0
        x[:, ::256] += 20.0
    else:
        raise ValueError(kind)
    return x.to(TDT[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["normal", "ties", "ascending", "descending", "zeros",
                                  "neg_inf", "stride"])
@pytest.mark.parametrize("V,k", [(7, 3), (64, 64), (300, 1), (1001, 17), (4096, 256),
                                 (32000, 64), (5000, 2048)])
def test_topk_shapes(vl, dtype, kind, V, k):
    x = topk_rows(kind, 5, V, dtype, V + k)
    ids, probs = run_topk(vl, x, k)
    oi, op = oracle.topk(to_host_bytes(x), k)
    check_topk(ids, probs, oi, op)


def test_topk_zipf_small(vl):
    for shared in (False, True):
        c = gi.topk_zipf(DEV, ntok=32, shared_perm=shared)
        ids, probs = run_topk(vl, c["teacher"], c["k"])
        oi, op = oracle.topk(to_host_bytes(c["teacher"]), c["k"])
        check_topk(ids, probs, oi, op)


def test_topk_long_rows(vl):
    # 2^20 values per row: vector indices and ids past 2^18 and 2^20
    x = gi.normal_logits(3, 1 << 20, 2.0, 78, DEV)
    ids, probs = run_topk(vl, x, 100)
    oi, op = oracle.topk(to_host_bytes(x), 100)
    check_topk(ids, probs, oi, op)


def test_topk_large_bf16_rows(vl):
    x = gi.normal_logits(8, 151936, 2.0, 77, DEV, torch.bfloat16)
    ids, probs = run_topk(vl, x, 256)
    oi, op = oracle.topk(to_host_bytes(x), 256)
    check_topk(ids, probs, oi, op)


# ------------------------------------------------------------ misaligned rows

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["ce", "kl", "topk"])
def test_misaligned_logits(vl, dtype, kind):
    ntok, V, k = 40, 4096, 48
    x = gi.normal_logits(ntok, V, 2.0, 31 + len(kind), DEV, TDT[dtype])
    if kind == "ce":
        assert_ce(vl, x, gi.uniform_labels(ntok, V, 32, DEV), (10, 2, 9), 1.0 / 28,
                  misalign=True)
    elif kind == "kl":
        assert_kl(vl, x, gi.distinct_ids(ntok, V, k, 33, DEV),
                  gi.softmax_probs(ntok, k, 1.5, 34, DEV), None, 0.25, misalign=True)
    else:
        ids, probs = run_topk(vl, offset_rows(x), k)
        oi, op = oracle.topk(to_host_bytes(x), k)
        check_topk(ids, probs, oi, op)


# ------------------------------------------------------------ slice accumulate

@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 1023, 1 << 20, 1000003])
@pytest.mark.parametrize("offset", [0, 1])
def test_slice_acc(vl, n, offset):
    g = torch.Generator(device=DEV)
    g.manual_seed(n + offset)
    a = torch.randn(n + offset, generator=g, device=DEV) * 1e3
    b = torch.randn(n + offset, generator=g, device=DEV) * 1e-3
    if n >= 8:
        a[offset:offset + 8] = torch.tensor([float("inf"), -0.0, 1e-40, 3.4e38, 1.0,
                                             2.0 ** -24, -1e-40, 5.0], device=DEV)
        b[offset:offset + 8] = torch.tensor([1.0, -0.0, 1e-40, 3.4e38, 2.0 ** -24, 1.0,
                                             2e-40, -5.0], device=DEV)
    dst, src = a[offset:], b[offset:]
    want = oracle.acc(dst.cpu().numpy(), src.cpu().numpy())
    vl.vl_slice_acc(dst, src)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
