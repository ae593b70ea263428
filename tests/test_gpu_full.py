"""Parity at the full workload sizes, in the launch configuration bench.py
times (the same C-ABI calls on the same shapes).  Every row's loss and
gradient at 4096 x 32000 and 8192 x 128256; at 16384 x 151936 every row's
loss, and the gradient of the first and last 1024 rows (the first and last
row of every workgroup's walk for any grid up to 1024 workgroups) plus
sampled rows between them, with whole-tensor invariants.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
from gen import inputs as gi
from gen.inputs import to_host_bytes
from tests.parity import (bf16_bits_to_f64, ce_target, check_grad, check_loss, check_topk,
                          dense_target)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def vl():
    import vocab_softmax_loss_amd as m
    assert torch.cuda.is_available()
    return m


def sample(ntok, n, seed, extra=()):
    r = np.random.default_rng(seed).choice(ntok, size=n, replace=False)
    return np.unique(np.concatenate([r, np.asarray(extra, dtype=np.int64)]))


def topk_invariants(x, ids, probs, k):
    """Whole-tensor checks valid at any size: ids distinct and in range,
    values non-increasing with ascending ids among equal values, probs
    positive-or-zero, non-increasing and summing to 1."""
    ids_l = ids.long()
    assert int(ids_l.min()) >= 0 and int(ids_l.max()) < x.shape[1]
    s = ids_l.sort(dim=1).values
    assert bool((s[:, 1:] != s[:, :-1]).all()), "repeated id in a row"
    v = x.gather(1, ids_l).float()
    dv = v[:, 1:] - v[:, :-1]
    assert bool((dv <= 0).all()), "values not non-increasing"
    tie = dv == 0
    assert bool(((ids_l[:, 1:] > ids_l[:, :-1]) | ~tie).all()), "tie not in id order"
    assert bool((probs >= 0).all())
    assert bool((probs[:, 1:] <= probs[:, :-1] * (1 + 1e-6)).all())
    assert float((probs.double().sum(dim=1) - 1).abs().max()) < 1e-5


def test_bench_step_full(vl):
    """The bench step exactly as bench.py times it (its inputs, calls and
    arguments, 4096 x 32000 float32): teacher top-k, KL against it, the
    prompt-masked CE, slice accumulate.  Every row against the oracle; the
    KL both against the GPU's top-k (stage-isolated) and end to end from
    the teacher bytes."""
    import bench
    x = bench.make_inputs(DEV)
    host = bench.host_copies(x)
    ntok, k = bench.NTOK, bench.K_TOPK
    ids = torch.empty((ntok, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((ntok, k), device=DEV)
    kl_loss = torch.empty(ntok, device=DEV)
    ce_loss = torch.empty(ntok, device=DEV)
    coef = 1024.0 / ntok
    vl.vl_topk_renorm(x["teacher"], k, ids, probs)
    vl.vl_kl_fwd_bwd(x["kl_student"], ids, probs, kl_loss, coef=coef)
    vl.vl_ce_fwd_bwd(x["ce_logits"], x["labels"], ce_loss, rng=x["rng"], scale=x["scale"])
    vl.vl_slice_acc(x["dh0"], x["dh1"])
    torch.cuda.synchronize()
    gi_ids = ids.cpu().numpy().view(np.uint32)
    gi_p = probs.cpu().numpy()
    kl_l, ce_l = kl_loss.cpu().numpy(), ce_loss.cpu().numpy()
    for r0 in range(0, ntok, 512):
        r1 = r0 + 512
        oi, op = oracle.topk(host["teacher"][r0:r1], k)
        check_topk(gi_ids[r0:r1], gi_p[r0:r1], oi, op)
        ol, olse, og = oracle.kl(host["kl_student"][r0:r1], gi_ids[r0:r1], gi_p[r0:r1],
                                 coef=coef)
        check_loss(kl_l[r0:r1], ol, "f32")
        check_grad(x["kl_student"][r0:r1].cpu().numpy(), og, "f32", coef,
                   tgt=dense_target(og.shape, gi_ids[r0:r1], gi_p[r0:r1], coef), lse=olse)
        el, _, _ = oracle.kl(host["kl_student"][r0:r1], oi, op.astype(np.float32), coef=coef,
                             want_grad=False)
        check_loss(kl_l[r0:r1], el, "f32", "KL end to end")
        ol, olse, og = oracle.ce(host["ce_logits"][r0:r1], host["labels"][r0:r1],
                                 rng=x["rng"], scale=x["scale"], row_index=np.arange(r0, r1))
        check_loss(ce_l[r0:r1], ol, "f32")
        check_grad(x["ce_logits"][r0:r1].cpu().numpy(), og, "f32", x["scale"],
                   tgt=ce_target(og.shape, host["labels"][r0:r1], x["scale"]), lse=olse)
    want = oracle.acc(host["dh0"], host["dh1"])
    assert np.array_equal(x["dh0"].cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_ce_lm_full(vl):
    """Cross-entropy, 8 x 512 tokens, V=32000, prompt mask: every row."""
    c = gi.ce_lm(DEV)
    x, lab, rng, scale = c["logits"], c["labels"], c["rng"], c["scale"]
    host = to_host_bytes(x)
    labh = lab.cpu().numpy()
    loss = torch.empty(x.shape[0], device=DEV)
    lse = torch.empty(x.shape[0], device=DEV)
    vl.vl_ce_fwd_bwd(x, lab, loss, lse, rng=rng, scale=scale)
    torch.cuda.synchronize()
    loss, lse = loss.cpu().numpy(), lse.cpu().numpy()
    for r0 in range(0, x.shape[0], 512):
        r1 = r0 + 512
        ol, olse, og = oracle.ce(host[r0:r1], labh[r0:r1], rng=rng, scale=scale,
                                 row_index=np.arange(r0, r1))
        check_loss(loss[r0:r1], ol, "f32")
        check_loss(lse[r0:r1], olse, "f32", "lse")
        check_grad(x[r0:r1].cpu().numpy(), og, "f32", scale,
                   tgt=ce_target(og.shape, labh[r0:r1], scale), lse=olse)


def test_ce_split_lm_full(vl):
    """The same configuration through the two-call CE (forward only, backward
    from the saved lse) and the device mean: every row, and the mean against
    the oracle's mean of the oracle's losses."""
    c = gi.ce_lm(DEV)
    x, lab, rng, scale = c["logits"], c["labels"], c["rng"], c["scale"]
    host = to_host_bytes(x)
    labh = lab.cpu().numpy()
    n = x.shape[0]
    loss = torch.empty(n, device=DEV)
    lse = torch.empty(n, device=DEV)
    mean = torch.empty(1, device=DEV)
    vl.vl_ce_fwd(x, lab, loss, lse, rng=rng)
    vl.vl_loss_mean(loss, mean, rng=rng)
    vl.vl_ce_bwd(x, lab, lse, rng=rng, scale=scale)
    torch.cuda.synchronize()
    loss_h, lse_h = loss.cpu().numpy(), lse.cpu().numpy()
    all_loss = np.empty(n)
    for r0 in range(0, n, 512):
        r1 = r0 + 512
        ol, olse, og = oracle.ce(host[r0:r1], labh[r0:r1], rng=rng, scale=scale,
                                 row_index=np.arange(r0, r1))
        all_loss[r0:r1] = ol
        check_loss(loss_h[r0:r1], ol, "f32")
        check_loss(lse_h[r0:r1], olse, "f32", "lse")
        check_grad(x[r0:r1].cpu().numpy(), og, "f32", scale,
                   tgt=ce_target(og.shape, labh[r0:r1], scale), lse=olse)
    # per-row losses within 1e-5 relative, so their mean is too
    want = all_loss.sum() / (8 * 384)
    assert abs(float(mean.cpu()[0]) - want) <= 1e-5 * abs(want)
    assert abs(float(mean.cpu()[0]) - oracle.loss_mean(loss_h, rng)) <= np.spacing(
        np.float32(want))


def test_topk_zipf_full(vl):
    """Teacher top-k, 4096 x 32000, k=64: every row."""
    c = gi.topk_zipf(DEV)
    t, k = c["teacher"], c["k"]
    ids = torch.empty((t.shape[0], k), dtype=torch.int32, device=DEV)
    probs = torch.empty((t.shape[0], k), device=DEV)
    vl.vl_topk_renorm(t, k, ids, probs)
    torch.cuda.synchronize()
    topk_invariants(t, ids, probs, k)
    oi, op = oracle.topk(to_host_bytes(t), k)
    check_topk(ids.cpu().numpy().view(np.uint32), probs.cpu().numpy(), oi, op)


def test_kl_large_full(vl):
    """Distillation KL, 8192 x 128256 float32, k=128: every row's loss, lse
    and gradient against the oracle, in chunks of 256 rows."""
    c = gi.kl_large(DEV)
    x, ids, probs, coef = c["logits"], c["ids"], c["probs"], c["coef"]
    ntok = x.shape[0]
    host = to_host_bytes(x)
    idh = ids.cpu().numpy()
    ph = probs.cpu().numpy()
    loss = torch.empty(ntok, device=DEV)
    lse = torch.empty(ntok, device=DEV)
    vl.vl_kl_fwd_bwd(x, ids, probs, loss, lse, coef=coef)
    torch.cuda.synchronize()
    loss_h, lse_h = loss.cpu().numpy(), lse.cpu().numpy()
    g_all = x.cpu().numpy()
    for r0 in range(0, ntok, 256):
        r1 = min(ntok, r0 + 256)
        ol, olse, og = oracle.kl(host[r0:r1], idh[r0:r1], ph[r0:r1], coef=coef)
        check_loss(loss_h[r0:r1], ol, "f32")
        check_loss(lse_h[r0:r1], olse, "f32", "lse")
        check_grad(g_all[r0:r1], og, "f32", coef,
                   tgt=dense_target(og.shape, idh[r0:r1], ph[r0:r1], coef), lse=olse,
                   what=f"grad rows {r0}-{r1}")


def test_kl_bf16_sliced_full(vl):
    """bf16 distillation at V=151936: teacher top-k (k=256) by the GPU, KL of
    the student against it, and the slice accumulate of two [16384][1024]
    float32 input gradients.  Top-k ids bit-exact on sampled rows and
    invariants on all; every row's loss against the oracle, both fed the
    GPU's top-k (stage-isolated) and end to end from the oracle's own
    top-k on sampled rows; the gradient of the first and last 1024 rows and
    of sampled rows between them."""
    c = gi.kl_bf16_sliced(DEV)
    x, t, k, coef = c["logits"], c["teacher"], c["k"], c["coef"]
    ntok = x.shape[0]
    rows = sample(ntok, 24, 51, extra=[0, ntok - 1])
    rows_t = torch.from_numpy(rows).to(DEV)
    th = to_host_bytes(t[rows_t])
    xh_all = to_host_bytes(x)

    ids = torch.empty((ntok, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((ntok, k), device=DEV)
    vl.vl_topk_renorm(t, k, ids, probs)
    torch.cuda.synchronize()
    topk_invariants(t, ids, probs, k)
    oi, op = oracle.topk(th, k)
    check_topk(ids[rows_t].cpu().numpy().view(np.uint32), probs[rows_t].cpu().numpy(), oi, op)

    loss = torch.empty(ntok, device=DEV)
    lse = torch.empty(ntok, device=DEV)
    vl.vl_kl_fwd_bwd(x, ids, probs, loss, lse, coef=coef)
    torch.cuda.synchronize()
    loss_h, lse_h = loss.cpu().numpy(), lse.cpu().numpy()
    idh = ids.cpu().numpy().view(np.uint32)
    ph = probs.cpu().numpy()
    # stage-isolated, every row's loss and lse: the oracle KL fed the GPU's
    # own ids and probs
    sl, slse, _ = oracle.kl(xh_all, idh, ph, coef=coef, want_grad=False)
    check_loss(loss_h, sl, "bf16", "KL from the GPU's top-k")
    check_loss(lse_h, slse, "bf16", "lse")
    # gradient rows: the first and last 1024 and sampled rows between them
    grows = np.unique(np.concatenate([np.arange(1024), np.arange(ntok - 1024, ntok),
                                      sample(ntok, 64, 52)]))
    g_all = to_host_bytes(x[torch.from_numpy(grows).to(DEV)])
    for i0 in range(0, len(grows), 256):
        sel = grows[i0:i0 + 256]
        _, olse, og = oracle.kl(xh_all[sel], idh[sel], ph[sel], coef=coef)
        check_grad(g_all[i0:i0 + 256], og, "bf16", coef,
                   tgt=dense_target(og.shape, idh[sel], ph[sel], coef), lse=olse,
                   what=f"gradient from the GPU's top-k, rows {sel[0]}-{sel[-1]}")
    # end to end on the sampled rows: the oracle's own top-k of the teacher bytes
    xh = xh_all[rows]
    ol, olse, og = oracle.kl(xh, oi, op.astype(np.float32), coef=coef)
    check_loss(loss_h[rows], ol, "bf16")
    check_grad(to_host_bytes(x[rows_t]), og, "bf16", coef,
               tgt=dense_target(og.shape, oi, op, coef), lse=olse)

    d0, d1 = c["dh0"], c["dh1"]
    want = oracle.acc(d0.cpu().numpy(), d1.cpu().numpy())
    vl.vl_slice_acc(d0, d1)
    torch.cuda.synchronize()
    assert np.array_equal(d0.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("chunk", [16384, 4096])
def test_head_kl_full(vl, chunk):
    """Vocabulary head, 16384 x 151936 x 1024 bf16, k=256, in one chunk of
    16384 rows (the bench configuration) and in chunks of 4096: sampled rows,
    chunk edges included, against the oracle on those rows (each row's loss
    and dx depend on that row alone).  Tolerances as in
    tests/test_gpu_head.py."""
    c = gi.head_inputs(16384, 151936, 1024, 256, 6001, DEV, torch.bfloat16)
    x, w, ids, probs = c["x"], c["w"], c["ids"], c["probs"]
    ntok, hs = x.shape
    V = w.shape[0]
    dx = torch.empty((ntok, hs), device=DEV)
    loss = torch.empty(ntok, device=DEV)
    scratch = torch.empty(vl.vl_head_scratch_bytes(chunk, V, hs), dtype=torch.uint8, device=DEV)
    vl.vl_head_kl(x, w, ids, probs, dx, loss, ntok, 1024.0, chunk, scratch)
    torch.cuda.synchronize()
    rows = sample(ntok, 12, 61, extra=(0, 4095, 4096, 8191, 12288, ntok - 1))
    xr = oracle.round_half(x[rows].cpu().numpy(), "bf16")
    wr = w.float().cpu().numpy().astype(np.float64)
    rl, rdx = oracle.head_kl(xr, wr, ids[rows].cpu().numpy(), probs[rows].cpu().numpy(), ntok,
                             1024.0)
    got_l = loss.cpu().numpy()[rows].astype(np.float64)
    got_dx = dx.cpu().numpy()[rows].astype(np.float64)
    assert np.isfinite(loss.cpu().numpy()).all() and bool(torch.isfinite(dx).all())
    assert (np.abs(got_l - rl) <= 1e-4 + 1e-5 * np.abs(rl)).all(), (got_l, rl)
    for i in range(len(rows)):
        e = np.linalg.norm(got_dx[i] - rdx[i]) / np.linalg.norm(rdx[i])
        assert e < 2.4e-2, (rows[i], e)
