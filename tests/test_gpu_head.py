"""The vocabulary head with the distillation KL (vl_head_kl) through the C
ABI against the float64 oracle (oracle.head_kl) on the same inputs, each side
rounding the hidden rows and the head weights to the head's half type
itself.  Needs an MI355X.

Tolerances, from the cortiq-engine head_kl test's own bounds:
  loss: relative L2 of the loss vector < 1e-4 (the page's bound), and each
        row within 1e-4 absolute + 1e-5 relative: the products of two half
        values are exact in float32, so the logits differ from the float64
        ones only by float32 accumulation over hs terms.
  dx:   relative L2 < 3e-3 for f16 (the page's bound), per row as well as
        over the tensor.  dx is formed from the gradient rounded once into
        the half type, so the error scales with that type's unit roundoff:
        bf16 (2^-8) gets the same bound in units of its roundoff as f16
        (2^-11) has, 8 x 3e-3 = 2.4e-2.
"""
import numpy as np
import pytest
import torch

import oracle
from gen import inputs as gi

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HALF = {"f16": torch.float16, "bf16": torch.bfloat16}
DX_TOL = {"f16": 3e-3, "bf16": 2.4e-2}


@pytest.fixture(scope="module")
def vl():
    import vocab_softmax_loss_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run_head(vl, x, w, ids, probs, total, gscale, chunk):
    ntok, hs = x.shape
    V = w.shape[0]
    dx = torch.full((ntok, hs), float("nan"), device=DEV)
    loss = torch.full((ntok,), float("nan"), device=DEV)
    nb = vl.vl_head_scratch_bytes(min(chunk, ntok), V, hs)
    scratch = torch.empty(nb, dtype=torch.uint8, device=DEV)
    vl.vl_head_kl(x, w, ids, probs, dx, loss, total, gscale, chunk, scratch)
    torch.cuda.synchronize()
    return loss.cpu().numpy().astype(np.float64), dx.cpu().numpy().astype(np.float64)


def rel_l2(got, want):
    return np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)


def check(loss, dx, rl, rdx, dtype):
    assert np.isfinite(loss).all() and np.isfinite(dx).all()
    assert rel_l2(loss, rl) < 1e-4, rel_l2(loss, rl)
    bad = np.nonzero(~(np.abs(loss - rl) <= 1e-4 + 1e-5 * np.abs(rl)))[0]
    assert bad.size == 0, (bad[:5], loss[bad[:5]], rl[bad[:5]])
    assert rel_l2(dx, rdx) < DX_TOL[dtype], rel_l2(dx, rdx)
    for t in range(dx.shape[0]):
        e = rel_l2(dx[t], rdx[t])
        assert e < DX_TOL[dtype], (t, e)


def oracle_for(x, w_half, ids, probs, total, gscale, dtype):
    """The oracle on the GPU's inputs: x rounded to the half type the way
    the oracle rounds it, the weights exactly as stored."""
    xr = oracle.round_half(x.cpu().numpy(), dtype)
    wr = w_half.float().cpu().numpy().astype(np.float64)  # exact widening
    return oracle.head_kl(xr, wr, ids.cpu().numpy(), probs.cpu().numpy(), total, gscale)


def test_head_page_case(vl):
    """The page test: V=1024, hs=256, 45 tokens, k=16, f16, chunks of 32."""
    c = gi.page_head_tiny()
    x = torch.from_numpy(c["x"]).to(DEV)
    w = torch.from_numpy(c["w"]).to(DEV).half()
    ids = torch.from_numpy(c["ids"]).to(DEV)
    probs = torch.from_numpy(c["probs"]).to(DEV)
    loss, dx = run_head(vl, x, w, ids, probs, c["total"], c["gscale"], c["chunk"])
    rl, rdx = oracle.head_kl(oracle.round_half(c["x"], "f16"), oracle.round_half(c["w"], "f16"),
                             c["ids"], c["probs"], c["total"], c["gscale"])
    check(loss, dx, rl, rdx, "f16")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("ntok,V,hs,k,chunk", [
    (50, 1000, 72, 7, 16),       # V and hs off every tile size; a ragged last chunk
    (33, 4096, 256, 64, 33),     # one chunk
    (70, 32000, 512, 64, 64),    # language-model vocabulary, two chunks
    (5, 151936, 128, 256, 4),    # the largest vocabulary, ragged
    (300, 2048, 128, 16, 300),   # two 256-row tiles of the product, the second ragged
    (9, 4096, 64, 300, 9),       # k above 256: the gradient pass reads the ids twice
    (7, 999, 64, 5, 4),          # V not a multiple of 4: the element path of the gradient
    (6, 500, 20, 4, 3),          # hs not a multiple of 8: hipBLASLt and the fused row kernel
])
def test_head_shapes(vl, dtype, ntok, V, hs, k, chunk):
    c = gi.head_inputs(ntok, V, hs, k, 3000 + V + hs, DEV, HALF[dtype])
    total, gscale = ntok + 3, 256.0
    loss, dx = run_head(vl, c["x"], c["w"], c["ids"], c["probs"], total, gscale, chunk)
    rl, rdx = oracle_for(c["x"], c["w"], c["ids"], c["probs"], total, gscale, dtype)
    check(loss, dx, rl, rdx, dtype)


def test_head_zero_rows_and_repeat(vl):
    """ntok = 0 is a no-op; two calls in a row agree (the scratch carries
    nothing between calls)."""
    c = gi.head_inputs(20, 2048, 64, 16, 3100, DEV)
    z = torch.empty((0, 64), device=DEV)
    vl.vl_head_kl(z, c["w"], torch.empty((0, 16), dtype=torch.int32, device=DEV),
                  torch.empty((0, 16), device=DEV), torch.empty((0, 64), device=DEV),
                  torch.empty(0, device=DEV), 1, 1.0, 8,
                  torch.empty(0, dtype=torch.uint8, device=DEV))
    a = run_head(vl, c["x"], c["w"], c["ids"], c["probs"], 20, 64.0, 8)
    b = run_head(vl, c["x"], c["w"], c["ids"], c["probs"], 20, 64.0, 8)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-6, atol=0)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-6, atol=1e-12)


def test_head_bad_id_and_padded_teacher(vl):
    """An id >= V with p > 0 makes that row's loss NaN and leaves the other
    rows as the oracle has them; a teacher list padded with a repeated id at
    probability 0 gives the oracle's result (those entries take no part)."""
    ntok, V, hs, k = 12, 3000, 64, 8
    c = gi.head_inputs(ntok, V, hs, k, 3200, DEV, torch.bfloat16)
    ids, probs = c["ids"].clone(), c["probs"].clone()
    ids[3, 2] = V          # out of range, p > 0
    ids[5, 6:] = ids[5, 0]  # padding: repeated id at probability 0
    probs[5, 6:] = 0.0
    total, gscale = ntok, 64.0
    loss, dx = run_head(vl, c["x"], c["w"], ids, probs, total, gscale, 8)
    assert np.isnan(loss[3])
    keep = [r for r in range(ntok) if r != 3]
    ids_ok = ids.clone()
    ids_ok[3, 2] = 0
    rl, rdx = oracle_for(c["x"], c["w"], ids_ok, probs, total, gscale, "bf16")
    assert np.isfinite(loss[keep]).all()
    assert (np.abs(loss[keep] - rl[keep]) <= 1e-4 + 1e-5 * np.abs(rl[keep])).all()
    for t in keep:
        assert rel_l2(dx[t], rdx[t]) < DX_TOL["bf16"], t


# ------------------------------------------------ the teacher side (vl_head_topk)

@pytest.mark.parametrize("hs", [64, 20])
def test_head_nan_weight_and_row(vl, hs):
    """A NaN head weight row makes every row's logits hold a NaN, and a NaN
    hidden row makes that row's logits all NaN: those rows' loss and dx are
    NaN, as the definition gives, and the other rows still match the oracle.
    hs = 64 runs the matrix-core product with its statistics records, 20 the
    library product and the row kernels."""
    ntok, V, k, chunk = 7, 999, 5, 4
    c = gi.head_inputs(ntok, V, hs, k, 8300 + hs, DEV, torch.float16)
    total, gscale = ntok, 64.0
    w = c["w"].clone()
    w[3] = float("nan")
    loss, dx = run_head(vl, c["x"], w, c["ids"], c["probs"], total, gscale, chunk)
    assert np.isnan(loss).all() and np.isnan(dx).all()
    x = c["x"].clone()
    x[2] = float("nan")
    loss, dx = run_head(vl, x, c["w"], c["ids"], c["probs"], total, gscale, chunk)
    assert np.isnan(loss[2]) and np.isnan(dx[2]).all()
    keep = np.array([r for r in range(ntok) if r != 2])
    rl, rdx = oracle_for(c["x"], c["w"], c["ids"], c["probs"], total, gscale, "f16")
    check(loss[keep], dx[keep], rl[keep], rdx[keep], "f16")


@pytest.mark.parametrize("hs", [64, 20])
def test_head_tune_then_plain(vl, hs):
    """vl_head_kl_tune, then vl_head_kl twice on the same shape: all three
    match the oracle, and the two plain calls, which run the tuned choice,
    agree bit for bit.  hs = 20 puts both products in hipBLASLt, hs = 64
    only the dx product."""
    ntok, V, k, chunk = 40, 3000, 8, 40
    c = gi.head_inputs(ntok, V, hs, k, 8400 + hs, DEV, torch.bfloat16)
    total, gscale = ntok, 128.0
    rl, rdx = oracle_for(c["x"], c["w"], c["ids"], c["probs"], total, gscale, "bf16")
    dx = torch.full((ntok, hs), float("nan"), device=DEV)
    loss = torch.full((ntok,), float("nan"), device=DEV)
    scratch = torch.empty(vl.vl_head_scratch_bytes(chunk, V, hs), dtype=torch.uint8, device=DEV)
    vl.vl_head_kl(c["x"], c["w"], c["ids"], c["probs"], dx, loss, total, gscale, chunk, scratch,
                  tune=True)
    torch.cuda.synchronize()
    check(loss.cpu().numpy().astype(np.float64), dx.cpu().numpy().astype(np.float64), rl, rdx,
          "bf16")
    a = run_head(vl, c["x"], c["w"], c["ids"], c["probs"], total, gscale, chunk)
    b = run_head(vl, c["x"], c["w"], c["ids"], c["probs"], total, gscale, chunk)
    check(a[0], a[1], rl, rdx, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_head_topk_tune(vl):
    """vl_head_topk_tune on a shape whose product runs in hipBLASLt (hs not a
    multiple of 8), on exact logits: the same ids and probabilities as the
    plain call and the oracle's ids."""
    ntok, V, hs, k = 30, 2000, 20, 16
    x, w = dyadic_head(ntok, V, hs, 8500, "bf16")
    scratch = torch.empty(vl.vl_head_topk_scratch_bytes(ntok, V, hs), dtype=torch.uint8,
                          device=DEV)
    out = []
    for tune in (True, False):
        ids = torch.empty((ntok, k), dtype=torch.int32, device=DEV)
        probs = torch.empty((ntok, k), device=DEV)
        vl.vl_head_topk(x, w, k, ids, probs, ntok, scratch, tune=tune)
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), probs.cpu().numpy()))
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])
    oi, _ = oracle.head_topk(x.cpu().numpy().astype(np.float64),
                             w.float().cpu().numpy().astype(np.float64), k)
    assert np.array_equal(out[0][0].view(np.uint32), oi)


def run_head_topk(vl, x, w, k, chunk):
    ntok, hs = x.shape
    V = w.shape[0]
    ids = torch.full((ntok, k), -1, dtype=torch.int32, device=DEV)
    probs = torch.full((ntok, k), float("nan"), device=DEV)
    nb = vl.vl_head_topk_scratch_bytes(min(chunk, ntok), V, hs)
    scratch = torch.empty(nb, dtype=torch.uint8, device=DEV)
    vl.vl_head_topk(x, w, k, ids, probs, chunk, scratch)
    torch.cuda.synchronize()
    return ids.cpu().numpy().view(np.uint32), probs.cpu().numpy().astype(np.float64)


def dyadic_head(ntok, V, hs, seed, dtype):
    """Hidden rows in quarters and head weights in eighths (both exact in
    f16 and bf16): every product and partial sum of a logit is exact in
    float32 for hs <= 64, so the GPU's float32 logits are the exact ones
    whatever the order of accumulation, and ties are common."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = torch.randint(-4, 5, (ntok, hs), generator=g, device=DEV).float() / 4
    w = (torch.randint(-8, 9, (V, hs), generator=g, device=DEV).float() / 8).to(HALF[dtype])
    return x, w


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("ntok,V,hs,k,chunk", [
    (37, 1000, 64, 64, 16),       # ragged last chunk
    (20, 32000, 32, 256, 20),     # one chunk
    (5, 151936, 48, 2048, 3),     # the largest vocabulary, the largest k
    (9, 7, 4, 7, 4),              # k = V
])
def test_head_topk_exact_logits(vl, dtype, ntok, V, hs, k, chunk):
    """Exact float32 logits: ids bit-exact against the oracle's head top-k
    (ties to the lower id), probabilities within 1e-5 relative."""
    x, w = dyadic_head(ntok, V, hs, 8000 + V, dtype)
    ids, probs = run_head_topk(vl, x, w, k, chunk)
    oi, op = oracle.head_topk(x.cpu().numpy().astype(np.float64),
                              w.float().cpu().numpy().astype(np.float64), k)
    np.testing.assert_array_equal(ids, oi)
    assert np.all(np.abs(probs - op) <= 1e-5 * np.abs(op) + 1e-12)


def check_near(ids, probs, s, eps, k, what):
    """ids/probs from float32 logits against the float64 logits s, where
    each float32 logit is within eps[t] of s: every id whose logit clears the
    oracle's k-th by more than 2 eps is chosen, every chosen id comes within
    2 eps of it, the chosen logits do not increase by more than 2 eps, and
    the probabilities are the renormalised softmax of the chosen logits."""
    n = s.shape[0]
    cols = np.arange(s.shape[1])
    for t in range(n):
        order = np.lexsort((cols, -s[t]))
        kth = s[t, order[k - 1]]
        got = ids[t].astype(np.int64)
        assert len(set(got.tolist())) == k, (what, t, "repeated id")
        must = order[s[t, order] > kth + 2 * eps[t]]
        assert set(must.tolist()) <= set(got.tolist()), (what, t, "a clear winner is missing")
        v = s[t, got]
        assert np.all(v >= kth - 2 * eps[t]), (what, t, "a chosen id is not near the top k")
        assert np.all(np.diff(v) <= 2 * eps[t]), (what, t, "not in descending order")
        e = np.exp(v - v[0])
        want = e / e.sum()
        assert np.all(np.abs(probs[t] - want) <= 1e-4 * want + 1e-12), (what, t)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_topk_random(vl, dtype):
    """N(0, 1) hidden rows and N(0, 1/hs) weights: the float32 logits carry
    accumulation error, bounded by hs 2^-24 sum_i |x_i w_i| per logit."""
    ntok, V, hs, k = 50, 32000, 512, 64
    c = gi.head_inputs(ntok, V, hs, 4, 8100, DEV, HALF[dtype])
    x, w = c["x"], c["w"]
    ids, probs = run_head_topk(vl, x, w, k, 32)
    xr = oracle.round_half(x.cpu().numpy(), dtype)
    wr = w.float().cpu().numpy().astype(np.float64)
    s = xr @ wr.T
    eps = hs * 2.0 ** -24 * (np.abs(xr) @ np.abs(wr).T).max(axis=1)
    check_near(ids, probs, s, eps, k, dtype)


@pytest.mark.slow
def test_head_topk_full(vl):
    """The teacher side at 16384 x 151936 x 1024 bf16, k = 256, in one
    chunk: sampled rows (chunk edges included) as in the random case, and
    invariants on every row."""
    ntok, V, hs, k = 16384, 151936, 1024, 256
    c = gi.head_inputs(ntok, V, hs, 4, 8200, DEV, torch.bfloat16)
    x, w = c["x"], c["w"]
    ids = torch.empty((ntok, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((ntok, k), device=DEV)
    scratch = torch.empty(vl.vl_head_topk_scratch_bytes(ntok, V, hs), dtype=torch.uint8,
                          device=DEV)
    vl.vl_head_topk(x, w, k, ids, probs, ntok, scratch)
    torch.cuda.synchronize()
    il = ids.long()
    assert int(il.min()) >= 0 and int(il.max()) < V
    srt = il.sort(dim=1).values
    assert bool((srt[:, 1:] != srt[:, :-1]).all())
    assert float((probs.double().sum(dim=1) - 1).abs().max()) < 1e-5
    rows = np.unique(np.concatenate([np.random.default_rng(62).choice(ntok, 12, replace=False),
                                     [0, ntok - 1]]))
    rt = torch.from_numpy(rows).to(DEV)
    xr = oracle.round_half(x[rt].cpu().numpy(), "bf16")
    wr = w.float().cpu().numpy().astype(np.float64)
    s = xr @ wr.T
    eps = hs * 2.0 ** -24 * (np.abs(xr) @ np.abs(wr).T).max(axis=1)
    check_near(ids[rt].cpu().numpy().view(np.uint32), probs[rt].cpu().numpy().astype(np.float64),
               s, eps, k, "full")
