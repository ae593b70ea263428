"""Calls on different streams are independent: the library keeps no state
between calls (no scratch, no counters), so the same calls issued on two
non-default streams at once give bit-identical results to the same calls
issued one after another.  Also checks that a call runs on the stream it
is given (the work is ordered after an event recorded on that stream).
Needs an MI355X."""
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


def make_work():
    V, k, n = 32000, 64, 1024
    teacher = gi.normal_logits(n, V, 2.0, 7001, DEV)
    student = gi.normal_logits(n, V, 2.0, 7002, DEV)
    c = gi.ce_lm(DEV, seed=7003, nseq=2)
    half = V // 2
    slices = [student[:, :half].contiguous(), student[:, half:].contiguous()]
    return dict(teacher=teacher, student=student, ce=c, slices=slices, k=k, n=n, half=half)


def run_all(vl, w, streams):
    """top-k then KL on streams[0]; CE and the sliced KL on streams[1]."""
    s0, s1 = streams
    n, k = w["n"], w["k"]
    ids = torch.empty((n, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((n, k), device=DEV)
    kl_loss = torch.empty(n, device=DEV)
    ce = w["ce"]
    ce_loss = torch.empty(ce["logits"].shape[0], device=DEV)
    x = w["student"].clone()
    ce_x = ce["logits"].clone()
    sl = [t.clone() for t in w["slices"]]
    parts = torch.empty((2, n, 4), device=DEV)
    s_loss = torch.empty(n, device=DEV)
    s_lse = torch.empty(n, device=DEV)
    fixed = torch.from_numpy(np.arange(n * k, dtype=np.int32).reshape(n, k) % 32000).to(DEV)
    fixed_p = torch.full((n, k), 1.0 / k, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s0):
        vl.vl_topk_renorm(w["teacher"], k, ids, probs)
        vl.vl_kl_fwd_bwd(x, ids, probs, kl_loss, coef=1.0 / n)
    with torch.cuda.stream(s1):
        vl.vl_ce_fwd_bwd(ce_x, ce["labels"], ce_loss, rng=ce["rng"], scale=ce["scale"])
        for i in range(2):
            vl.vl_kl_slice_fwd(sl[i], i * w["half"], fixed, fixed_p, parts[i])
        vl.vl_kl_slice_merge(parts, s_loss, s_lse)
        for i in range(2):
            vl.vl_kl_slice_bwd(sl[i], i * w["half"], fixed, fixed_p, s_lse, coef=0.5)
    torch.cuda.synchronize()
    out = [ids, probs, kl_loss, x, ce_loss, ce_x, s_loss, s_lse] + sl
    return [to_host_bytes(t) if t.dtype != torch.int32 else t.cpu().numpy() for t in out]


def test_two_streams_match_one_stream(vl):
    w = make_work()
    d = torch.cuda.current_stream()
    seq = run_all(vl, w, (d, d))
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        par = run_all(vl, w, (a, b))
        for i, (x, y) in enumerate(zip(seq, par)):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"output {i} differs"


def test_call_runs_on_the_given_stream(vl):
    """The CE call is issued on stream s after s waits for an event that a
    long top-k on another stream records: the CE reads logits that the
    other stream writes just before that event, so a call that ignored s
    would read the old values."""
    n, V = 512, 32000
    big = gi.normal_logits(4096, V, 2.0, 7101, DEV)
    bids = torch.empty((4096, 64), dtype=torch.int32, device=DEV)
    bp = torch.empty((4096, 64), device=DEV)
    x = torch.zeros((n, V), device=DEV)
    src = gi.normal_logits(n, V, 2.0, 7102, DEV)
    lab = gi.uniform_labels(n, V, 7103, DEV)
    loss = torch.empty(n, device=DEV)
    want = torch.empty(n, device=DEV)
    vl.vl_ce_fwd(src, lab, want)
    torch.cuda.synchronize()
    s_prod, s = torch.cuda.Stream(), torch.cuda.Stream()
    ev = torch.cuda.Event()
    with torch.cuda.stream(s_prod):
        for _ in range(4):
            vl.vl_topk_renorm(big, 64, bids, bp)
        x.copy_(src)
        ev.record(s_prod)
    s.wait_event(ev)
    vl.vl_ce_fwd(x, lab, loss, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(loss, want)
