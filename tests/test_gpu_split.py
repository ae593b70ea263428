"""The split-row calls (vl_ce_fwd_bwd_ws, vl_kl_fwd_bwd_ws) against the
float64 oracle, through the C ABI: rows split over 2, 4 and 8 workgroups,
float32 and bf16, with several rows per workgroup group and a loss range,
plus edge cases.  Tolerances are in tests/parity.py.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
from gen import inputs as gi
from gen.inputs import to_host_bytes
from tests.parity import ce_target, check_grad, check_loss, dense_target

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def vl():
    import vocab_softmax_loss_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def ws(vl):
    return torch.empty(vl.vl_split_workspace_bytes(), dtype=torch.uint8, device=DEV)


def dname(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def parts(dtype, V):
    """Parts the library splits a row into (mirrors its launch table: a
    part is at most 1024 x 8 float32 or 512 x 7 bf16 16-byte vectors; bf16
    rows of up to 155648 values stay whole), 0 when not split."""
    n = 4 if dtype == "f32" else 8
    per = 1024 * 8 if dtype == "f32" else 512 * 7
    nvec = V // n
    if nvec <= (8192 if dtype == "f32" else 19456):
        return 0
    s = max(2, -(-nvec // per))
    return s if s <= 16 else 0


def rows_for(dtype, S):
    """Three rows per workgroup group (float32: one workgroup per CU, bf16:
    two, on 256 CUs; S per group, groups in multiples of 8) and a few more,
    so every group walks several rows."""
    per_cu = 1 if dtype == "f32" else 2
    groups = per_cu * 256 // S // 8 * 8
    return 3 * groups + 5


def run_ce_ws(vl, x, lab, rng, scale, ws):
    out = x.clone()
    n = x.shape[0]
    loss = torch.full((n,), float("nan"), device=DEV)
    lse = torch.full((n,), float("nan"), device=DEV)
    vl.vl_ce_fwd_bwd_ws(out, lab, loss, ws, lse, rng=rng, scale=scale)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy(), out


def run_kl_ws(vl, x, ids, probs, rng, coef, ws):
    out = x.clone()
    n = x.shape[0]
    loss = torch.full((n,), float("nan"), device=DEV)
    lse = torch.full((n,), float("nan"), device=DEV)
    vl.vl_kl_fwd_bwd_ws(out, ids, probs, loss, ws, lse, rng=rng, coef=coef)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy(), out


def check_all(kind, host, got, loss, lse, tg, probs, rng, coef, dtype):
    """Every row against the oracle, in chunks of about 2^25 values."""
    n, V = host.shape
    step = max(1, (1 << 25) // V)
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        ri = np.arange(r0, r1)
        g = to_host_bytes(got[r0:r1])
        if kind == "ce":
            ol, olse, og = oracle.ce(host[r0:r1], tg[r0:r1], rng=rng, scale=coef, row_index=ri)
            tgt = ce_target(og.shape, tg[r0:r1], coef)
        else:
            ol, olse, og = oracle.kl(host[r0:r1], tg[r0:r1], probs[r0:r1], rng=rng, coef=coef,
                                     row_index=ri)
            tgt = dense_target(og.shape, tg[r0:r1], probs[r0:r1], coef)
        check_loss(loss[r0:r1], ol, dtype, f"loss rows {r0}-{r1}")
        check_loss(lse[r0:r1], olse, dtype, f"lse rows {r0}-{r1}")
        check_grad(g, og, dtype, coef, f"grad rows {r0}-{r1}", tgt=tgt, lse=olse)


SHAPES = [("f32", 32772), ("f32", 65540), ("f32", 128256), ("f32", 262144), ("f32", 524288),
          ("bf16", 155656), ("bf16", 200000), ("bf16", 311296), ("bf16", 458752)]


def test_shapes_cover_the_splits():
    got = [(d, parts(d, V)) for d, V in SHAPES]
    assert got == [("f32", 2), ("f32", 3), ("f32", 4), ("f32", 8), ("f32", 16),
                   ("bf16", 6), ("bf16", 7), ("bf16", 11), ("bf16", 16)]


@pytest.mark.parametrize("kind", ["ce", "kl"])
@pytest.mark.parametrize("dtype,V", SHAPES)
def test_split_rows_with_range(vl, ws, kind, dtype, V):
    S = parts(dtype, V)
    ntok = rows_for(dtype, S)
    print(f"split {kind} {dtype} V={V} S={S} ntok={ntok}", flush=True)
    x = gi.normal_logits(ntok, V, 2.5, 5000 + V, DEV, TDT[dtype])
    rng = (7, 1, 6)
    coef = 1.0 / 300
    if kind == "ce":
        tg = gi.uniform_labels(ntok, V, 5100 + V, DEV)
        loss, lse, g = run_ce_ws(vl, x, tg, rng, coef, ws)
        probs = None
    else:
        k = 256 if V < 500000 else 64
        tg = gi.distinct_ids(ntok, V, k, 5200 + V, DEV)
        pt = gi.softmax_probs(ntok, k, 1.5, 5300 + V, DEV)
        loss, lse, g = run_kl_ws(vl, x, tg, pt, rng, coef, ws)
        probs = pt.cpu().numpy()
    check_all(kind, to_host_bytes(x), g, loss, lse, tg.cpu().numpy(), probs, rng, coef, dtype)


@pytest.mark.parametrize("dtype,V", [("f32", 128256), ("bf16", 200000)])
def test_split_matches_the_unsplit_call(vl, ws, dtype, V):
    """The same rows through vl_kl_fwd_bwd and vl_kl_fwd_bwd_ws: losses and
    lse within float32 rounding of each other, gradients within the
    gradient tolerance of each other."""
    ntok, k = 300, 128
    x = gi.normal_logits(ntok, V, 2.0, 5400 + V, DEV, TDT[dtype])
    ids = gi.distinct_ids(ntok, V, k, 5401, DEV)
    probs = gi.softmax_probs(ntok, k, 1.5, 5402, DEV)
    a = x.clone()
    la = torch.empty(ntok, device=DEV)
    sa = torch.empty(ntok, device=DEV)
    vl.vl_kl_fwd_bwd(a, ids, probs, la, sa, coef=0.125)
    lb, sb, b = run_kl_ws(vl, x, ids, probs, None, 0.125, ws)
    la, sa = la.cpu().numpy(), sa.cpu().numpy()
    assert np.all(np.abs(lb - la) <= 1e-5 * np.abs(la) + 1e-6)
    assert np.all(np.abs(sb - sa) <= 4e-7 * np.abs(sa))
    ga = a.float().cpu().numpy().astype(np.float64)
    gb = b.float().cpu().numpy().astype(np.float64)
    if dtype == "f32":
        assert np.all(np.abs(gb - ga) <= 1e-6)
    rel = np.linalg.norm(gb - ga, axis=1) / np.linalg.norm(ga, axis=1)
    assert rel.max() < (1e-5 if dtype == "f32" else 4e-3), rel.max()


@pytest.mark.parametrize("dtype,V", [("f32", 128256), ("bf16", 200000)])
@pytest.mark.parametrize("ntok", [1, 5, 37])
def test_split_fewer_rows_than_groups(vl, ws, dtype, V, ntok):
    x = gi.normal_logits(ntok, V, 2.0, 5500 + ntok, DEV, TDT[dtype])
    lab = gi.uniform_labels(ntok, V, 5501 + ntok, DEV)
    loss, lse, g = run_ce_ws(vl, x, lab, None, 0.5, ws)
    check_all("ce", to_host_bytes(x), g, loss, lse, lab.cpu().numpy(), None, None, 0.5, dtype)


@pytest.mark.parametrize("dtype,V", [("f32", 128256), ("bf16", 200000)])
def test_split_nan_logit(vl, ws, dtype, V):
    """A NaN logit in one part of a split row makes that row's lse and loss
    NaN (the part's sum is NaN and the exchange keeps it); the other rows
    come out exactly as without it."""
    ntok, k = 9, 16
    x = gi.normal_logits(ntok, V, 2.0, 5650, DEV, TDT[dtype])
    ids = gi.distinct_ids(ntok, V, k, 5651, DEV)
    probs = gi.softmax_probs(ntok, k, 1.5, 5652, DEV)
    l0, s0, g0 = run_kl_ws(vl, x, ids, probs, None, 0.25, ws)
    y = x.clone()
    y[4, V - 7] = float("nan")
    l1, s1, g1 = run_kl_ws(vl, y, ids, probs, None, 0.25, ws)
    assert np.isnan(l1[4]) and np.isnan(s1[4])
    keep = [r for r in range(ntok) if r != 4]
    assert np.array_equal(l1[keep], l0[keep]) and np.array_equal(s1[keep], s0[keep])
    assert torch.equal(g1[keep], g0[keep])


def test_split_all_rows_outside_the_range(vl, ws):
    V = 128256
    x = gi.normal_logits(40, V, 2.0, 5600, DEV)
    lab = gi.uniform_labels(40, V, 5601, DEV)
    loss, lse, g = run_ce_ws(vl, x, lab, (8, 3, 3), 1.0, ws)
    assert not loss.any() and not lse.any() and not bool(g.any())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_many_teacher_entries_and_padding(vl, ws, dtype):
    """k = 700 (threads take several entries each), ids packed into few
    16-byte vectors on some rows, and the tail of every row padded with a
    repeated id at probability 0."""
    V, ntok, k = 65544, 200, 700
    x = gi.normal_logits(ntok, V, 2.0, 5700, DEV, TDT[dtype])
    ids = gi.distinct_ids(ntok, V, k, 5701, DEV)
    gen = torch.Generator()
    gen.manual_seed(5703)
    for r in range(0, ntok, 3):  # 16 consecutive ids (two to four 16-byte vectors) first
        perm = torch.randperm(V, generator=gen)
        blk = int(perm[0]) // 16 * 16
        rest = perm[perm // 16 != blk // 16][:k - 16]
        ids[r] = torch.cat([blk + torch.arange(16), rest]).to(ids.dtype).to(DEV)
    probs = gi.softmax_probs(ntok, k, 1.5, 5702, DEV)
    probs[:, 600:] = 0.0
    ids[:, 600:] = ids[:, 1:2]
    probs /= probs.sum(dim=1, keepdim=True)
    for r in range(0, ntok, 3):
        assert torch.unique(ids[r, :600]).numel() == 600
    loss, lse, g = run_kl_ws(vl, x, ids, probs, None, 1.0 / ntok, ws)
    check_all("kl", to_host_bytes(x), g, loss, lse, ids.cpu().numpy(), probs.cpu().numpy(),
              None, 1.0 / ntok, dtype)


def test_split_invalid_ids_give_nan_loss_only(vl, ws):
    V = 128256
    x = gi.normal_logits(6, V, 2.0, 5800, DEV)
    ids = gi.distinct_ids(6, V, 8, 5801, DEV)
    ids[2, 5] = V + 3
    probs = torch.full((6, 8), 0.125, device=DEV)
    loss, lse, g = run_kl_ws(vl, x, ids, probs, None, 1.0, ws)
    assert np.isnan(loss[2]) and np.isfinite(np.delete(loss, 2)).all()
    keep = [0, 1, 3, 4, 5]
    idh, ph = ids.cpu().numpy()[keep], probs.cpu().numpy()[keep]
    ol, olse, og = oracle.kl(to_host_bytes(x)[keep], idh, ph, coef=1.0)
    check_loss(loss[keep], ol, "f32")
    check_grad(to_host_bytes(g)[keep], og, "f32", 1.0, tgt=dense_target(og.shape, idh, ph, 1.0),
               lse=olse)


def test_split_workspace_contents_do_not_matter(vl):
    """A workspace full of ones (a stale mailbox) and the same workspace
    reused for a second, smaller call: both match the oracle."""
    wsx = torch.full((vl.vl_split_workspace_bytes(),), 255, dtype=torch.uint8, device=DEV)
    for ntok, seed in ((300, 5900), (17, 5901)):
        V = 200000
        x = gi.normal_logits(ntok, V, 2.0, seed, DEV, torch.bfloat16)
        ids = gi.distinct_ids(ntok, V, 64, seed + 1, DEV)
        probs = gi.softmax_probs(ntok, 64, 1.5, seed + 2, DEV)
        loss, lse, g = run_kl_ws(vl, x, ids, probs, None, 0.25, wsx)
        check_all("kl", to_host_bytes(x), g, loss, lse, ids.cpu().numpy(),
                  probs.cpu().numpy(), None, 0.25, "bf16")


def test_split_short_or_unaligned_rows_take_the_unsplit_kernels(vl, ws):
    """Rows the split does not take (short, bf16 rows one workgroup holds,
    or not 16-byte aligned) give the unsplit call's bits exactly."""
    for V, off, dt in ((32000, 0, torch.float32), (151936, 0, torch.bfloat16),
                       (128256, 1, torch.float32)):
        ntok = 9
        base = gi.normal_logits(ntok * V + 1, 1, 2.0, 6000 + V, DEV, dt).view(-1)
        x = base[off:off + ntok * V].view(ntok, V)
        lab = gi.uniform_labels(ntok, V, 6001, DEV)
        a, b = x.clone(), x.clone()
        if off:
            a = base.clone()[off:off + ntok * V].view(ntok, V)
            b = base.clone()[off:off + ntok * V].view(ntok, V)
        la, lb = torch.empty(ntok, device=DEV), torch.empty(ntok, device=DEV)
        vl.vl_ce_fwd_bwd(a, lab, la, scale=0.5)
        vl.vl_ce_fwd_bwd_ws(b, lab, lb, ws, scale=0.5)
        torch.cuda.synchronize()
        assert torch.equal(la, lb) and torch.equal(a, b)
