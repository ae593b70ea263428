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
