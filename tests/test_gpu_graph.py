"""The calls inside a captured HIP graph (torch.cuda.CUDAGraph): the library
launches kernels only on the given stream and uses no memset, no allocation
and no synchronisation, so a captured sequence replays to the same bits as
the same sequence run eagerly, replay after replay, with the program's own
eager work and synchronisations between replays.  Needs an MI355X."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from gen.inputs import to_host_bytes

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def vl():
    import vocab_softmax_loss_amd as m
    assert torch.cuda.is_available()
    return m


def test_graph_replays_match_eager(vl):
    n, V, k, hs = 512, 32000, 64, 1024
    half = V // 2
    teacher = gi.normal_logits(n, V, 2.0, 8001, DEV)
    student_src = gi.normal_logits(n, V, 2.0, 8002, DEV)
    c = gi.ce_lm(DEV, seed=8003, nseq=1)
    ce_src, labels, rng, scale = c["logits"], c["labels"], c["rng"], c["scale"]
    g = torch.Generator(device=DEV)
    g.manual_seed(8004)
    d0_src = torch.randn((n, hs), generator=g, device=DEV)
    d1 = torch.randn((n, hs), generator=g, device=DEV)

    # static buffers the graph reads and writes
    student = torch.empty_like(student_src)
    ce_x = torch.empty_like(ce_src)
    sl = [torch.empty((n, half), device=DEV) for _ in range(2)]
    d0 = torch.empty_like(d0_src)
    ids = torch.empty((n, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((n, k), device=DEV)
    kl_loss = torch.empty(n, device=DEV)
    ce_loss = torch.empty(ce_src.shape[0], device=DEV)
    parts = torch.empty((2, n, 4), device=DEV)
    s_loss = torch.empty(n, device=DEV)
    s_lse = torch.empty(n, device=DEV)
    outs = [ids, probs, kl_loss, student, ce_loss, ce_x, parts, s_loss, s_lse, sl[0], sl[1], d0]

    def reset():
        student.copy_(student_src)
        ce_x.copy_(ce_src)
        sl[0].copy_(student_src[:, :half])
        sl[1].copy_(student_src[:, half:])
        d0.copy_(d0_src)

    def step():
        vl.vl_topk_renorm(teacher, k, ids, probs)
        vl.vl_kl_fwd_bwd(student, ids, probs, kl_loss, coef=1.0 / n)
        vl.vl_ce_fwd_bwd(ce_x, labels, ce_loss, rng=rng, scale=scale)
        for i in range(2):
            vl.vl_kl_slice_fwd(sl[i], i * half, ids, probs, parts[i])
        vl.vl_kl_slice_merge(parts, s_loss, s_lse)
        for i in range(2):
            vl.vl_kl_slice_bwd(sl[i], i * half, ids, probs, s_lse, coef=1.0 / n)
        vl.vl_slice_acc(d0, d1)

    def snapshot():
        torch.cuda.synchronize()
        return [to_host_bytes(t) if t.dtype != torch.int32 else t.cpu().numpy() for t in outs]

    reset()
    step()
    ref = snapshot()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in outs:
            t.zero_()  # stale results must not survive a replay
        reset()
        graph.replay()
        got = snapshot()
        for i, (x, y) in enumerate(zip(ref, got)):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
                f"replay {rep}: output {i} differs from the eager run"
        # eager work of the program's own between replays
        step()
        torch.cuda.synchronize()


def test_split_calls_under_capture_run_whole_rows(vl):
    """The workspace and no-allocation calls inside a captured graph: a
    split is one cooperative launch, which a capture does not take, so they
    run the rows whole -- every replay gives the unsplit call's bits."""
    n, V, k = 96, 128256, 64
    src = gi.normal_logits(n, V, 2.0, 8101, DEV)
    ids = gi.distinct_ids(n, V, k, 8102, DEV)
    probs = gi.softmax_probs(n, k, 1.5, 8103, DEV)
    ws = torch.empty(vl.vl_split_workspace_bytes(), dtype=torch.uint8, device=DEV)
    ref = src.clone()
    ref_loss = torch.empty(n, device=DEV)
    vl.vl_kl_fwd_bwd(ref, ids, probs, ref_loss, coef=1.0 / n)
    a, b = torch.empty_like(src), torch.empty_like(src)
    la, lb = torch.empty(n, device=DEV), torch.empty(n, device=DEV)

    def step():
        vl.vl_kl_fwd_bwd_ws(a, ids, probs, la, ws, coef=1.0 / n)
        vl.vl_kl_fwd_bwd_noalloc(b, ids, probs, lb, coef=1.0 / n)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        a.copy_(src)
        b.copy_(src)
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    a.copy_(src)
    b.copy_(src)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        la.zero_()
        lb.zero_()
        a.copy_(src)
        b.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        for t, lt in ((a, la), (b, lb)):
            assert torch.equal(t, ref) and torch.equal(lt, ref_loss), f"replay {rep}"
        step()  # eager, split, between replays
        torch.cuda.synchronize()
