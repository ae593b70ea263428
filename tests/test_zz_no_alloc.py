"""The KL entry point that allocates nothing (vl_kl_fwd_bwd_noalloc, whose
split rows exchange through the library's own device array) against the
workspace entry point it is a variant of (vl_kl_fwd_bwd_ws), through the C
ABI: two calls in a row, the second on a smaller input (fewer rows, and
rows split into fewer parts), each bit for bit the workspace call's result
and within the oracle's tolerances.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
from gen import inputs as gi
from gen.inputs import to_host_bytes
from tests.parity import check_grad, check_loss, dense_target

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def vl():
    import vocab_softmax_loss_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run(vl, fn, x, ids, probs, rng, coef, ws=None):
    out = x.clone()
    n = x.shape[0]
    loss = torch.full((n,), float("nan"), device=DEV)
    lse = torch.full((n,), float("nan"), device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    if ws is None:
        fn(out, ids, probs, loss, lse, rng=rng, coef=coef)
    else:
        fn(out, ids, probs, loss, ws, lse, rng=rng, coef=coef)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(DEV) == before
    return loss, lse, out


@pytest.mark.parametrize("dtype,calls", [
    (torch.float32, [(300, 128256, 64), (40, 65540, 16)]),    # 4 parts, then 3
    (torch.bfloat16, [(200, 200000, 64), (33, 160008, 8)]),   # 7 parts, then 6
])
def test_noalloc_matches_the_workspace_call(vl, dtype, calls):
    ws = torch.empty(vl.vl_split_workspace_bytes(), dtype=torch.uint8, device=DEV)
    dname = "bf16" if dtype == torch.bfloat16 else "f32"
    for i, (ntok, V, k) in enumerate(calls):
        print(f"no-alloc call {i}: {dname} ntok={ntok} V={V} k={k}", flush=True)
        x = gi.normal_logits(ntok, V, 2.0, 7000 + V, DEV, dtype)
        ids = gi.distinct_ids(ntok, V, k, 7001 + V, DEV)
        probs = gi.softmax_probs(ntok, k, 1.5, 7002 + V, DEV)
        rng = (9, 1, 8) if i == 0 else None
        coef = 1.0 / ntok
        la, sa, ga = run(vl, vl.vl_kl_fwd_bwd_noalloc, x, ids, probs, rng, coef)
        lb, sb, gb = run(vl, vl.vl_kl_fwd_bwd_ws, x, ids, probs, rng, coef, ws)
        assert torch.equal(la, lb) and torch.equal(sa, sb) and torch.equal(ga, gb)
        idh, ph = ids.cpu().numpy(), probs.cpu().numpy()
        ri = np.arange(ntok)
        ol, olse, og = oracle.kl(to_host_bytes(x), idh, ph, rng=rng, coef=coef, row_index=ri)
        check_loss(la.cpu().numpy(), ol, dname)
        check_loss(sa.cpu().numpy(), olse, dname, "lse")
        check_grad(to_host_bytes(ga), og, dname, coef, tgt=dense_target(og.shape, idh, ph, coef),
                   lse=olse)
