"""The C ABI on the CPU: libvl.so loads, exports every function include/vl.h
declares, and rejects invalid arguments on the host before any GPU work.
No call here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vl.h")

VL_OK, VL_EINVAL, VL_EDTYPE, VL_ELAUNCH = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    import vocab_softmax_loss_amd as vl
    return vl._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vl_[a-z_]+)\s*\(", text)))


def test_header_declares_the_calls():
    assert declared_functions() == sorted(
        ["vl_ce_fwd_bwd", "vl_ce_fwd", "vl_ce_bwd", "vl_loss_mean", "vl_kl_fwd_bwd",
         "vl_topk_renorm", "vl_slice_acc", "vl_head_scratch_bytes", "vl_head_kl",
         "vl_kl_slice_fwd", "vl_kl_slice_merge", "vl_kl_slice_bwd", "vl_strerror",
         "vl_split_workspace_bytes", "vl_ce_fwd_bwd_ws", "vl_kl_fwd_bwd_ws",
         "vl_kl_fwd_bwd_noalloc", "vl_head_topk_scratch_bytes", "vl_head_topk",
         "vl_head_kl_tune", "vl_head_topk_tune"])


def test_library_exports_every_declared_function(lib):
    raw = ctypes.CDLL(lib._name)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_strerror(lib):
    for st in (VL_OK, VL_EINVAL, VL_EDTYPE, VL_ELAUNCH, 7):
        assert lib.vl_strerror(st)
    assert lib.vl_strerror(VL_EDTYPE) != lib.vl_strerror(VL_EINVAL)


# A non-null pointer that is never dereferenced: every call below fails its
# host checks (or is a no-op) before touching it.
P = ctypes.c_void_p(0x1000)


def ce(lib, **kw):
    a = dict(logits=P, dtype=0, labels=P, loss=P, lse=None, ntok=4, V=10, rng=None,
             scale=1.0, stream=None)
    a.update(kw)
    return lib.vl_ce_fwd_bwd(a["logits"], a["dtype"], a["labels"], a["loss"], a["lse"],
                             a["ntok"], a["V"], a["rng"], a["scale"], a["stream"])


def kl(lib, **kw):
    a = dict(logits=P, dtype=0, ids=P, probs=P, k=2, loss=P, lse=None, ntok=4, V=10,
             rng=None, coef=1.0, stream=None)
    a.update(kw)
    return lib.vl_kl_fwd_bwd(a["logits"], a["dtype"], a["ids"], a["probs"], a["k"],
                             a["loss"], a["lse"], a["ntok"], a["V"], a["rng"], a["coef"],
                             a["stream"])


def rng(seq_len, start, end):
    import vocab_softmax_loss_amd as vl
    return ctypes.byref(vl.vl_range(seq_len, start, end))


def test_ce_host_checks(lib):
    assert ce(lib, dtype=2) == VL_EDTYPE
    assert ce(lib, dtype=-1) == VL_EDTYPE
    assert ce(lib, V=0) == VL_EINVAL
    assert ce(lib, V=1 << 31) == VL_EINVAL
    assert ce(lib, ntok=-1) == VL_EINVAL
    assert ce(lib, ntok=1 << 62, V=1 << 20) == VL_EINVAL  # ntok*V overflows
    assert ce(lib, logits=None) == VL_EINVAL
    assert ce(lib, labels=None) == VL_EINVAL
    assert ce(lib, loss=None) == VL_EINVAL
    assert ce(lib, rng=rng(0, 0, 0)) == VL_EINVAL
    assert ce(lib, rng=rng(8, 5, 4)) == VL_EINVAL
    assert ce(lib, rng=rng(8, -1, 4)) == VL_EINVAL
    assert ce(lib, rng=rng(8, 0, 9)) == VL_EINVAL
    # ntok == 0 is a no-op, even with null pointers
    assert ce(lib, ntok=0, logits=None, labels=None, loss=None) == VL_OK


def test_ce_split_host_checks(lib):
    fwd, bwd = lib.vl_ce_fwd, lib.vl_ce_bwd
    assert fwd(P, 2, P, P, None, 4, 10, None, None) == VL_EDTYPE
    assert fwd(P, 0, P, P, None, 4, 0, None, None) == VL_EINVAL
    assert fwd(P, 0, P, P, None, -1, 10, None, None) == VL_EINVAL
    assert fwd(None, 0, P, P, None, 4, 10, None, None) == VL_EINVAL
    assert fwd(P, 0, None, P, None, 4, 10, None, None) == VL_EINVAL
    assert fwd(P, 0, P, None, None, 4, 10, None, None) == VL_EINVAL
    assert fwd(P, 0, P, P, None, 4, 10, rng(4, 3, 2), None) == VL_EINVAL
    assert fwd(None, 0, None, None, None, 0, 10, None, None) == VL_OK
    assert bwd(P, 5, P, P, 4, 10, None, 1.0, None) == VL_EDTYPE
    assert bwd(P, 0, P, P, 4, 1 << 31, None, 1.0, None) == VL_EINVAL
    assert bwd(None, 0, P, P, 4, 10, None, 1.0, None) == VL_EINVAL
    assert bwd(P, 0, None, P, 4, 10, None, 1.0, None) == VL_EINVAL
    assert bwd(P, 0, P, None, 4, 10, None, 1.0, None) == VL_EINVAL  # lse is required
    assert bwd(P, 0, P, P, 4, 10, rng(0, 0, 0), 1.0, None) == VL_EINVAL
    assert bwd(None, 1, None, None, 0, 10, None, 1.0, None) == VL_OK


def test_loss_mean_host_checks(lib):
    f = lib.vl_loss_mean
    assert f(P, -1, None, P, None) == VL_EINVAL
    assert f(P, 4, None, None, None) == VL_EINVAL
    assert f(None, 4, None, P, None) == VL_EINVAL
    assert f(P, 4, rng(4, 2, 5), P, None) == VL_EINVAL
    assert f(P, 4, rng(0, 0, 0), P, None) == VL_EINVAL


def test_kl_host_checks(lib):
    assert kl(lib, dtype=3) == VL_EDTYPE
    assert kl(lib, k=0) == VL_EINVAL
    assert kl(lib, k=11) == VL_EINVAL  # k > V
    assert kl(lib, V=(1 << 19) + 1, k=4) == VL_EINVAL  # two V-bit bitmaps exceed LDS
    assert kl(lib, ids=None) == VL_EINVAL
    assert kl(lib, probs=None) == VL_EINVAL
    assert kl(lib, loss=None) == VL_EINVAL
    assert kl(lib, rng=rng(4, 3, 2)) == VL_EINVAL
    assert kl(lib, ntok=0, logits=None) == VL_OK


def test_topk_host_checks(lib):
    f = lib.vl_topk_renorm
    assert f(P, 9, 4, 10, 2, P, P, None) == VL_EDTYPE
    assert f(P, 0, 4, 10, 0, P, P, None) == VL_EINVAL
    assert f(P, 0, 4, 10, 11, P, P, None) == VL_EINVAL  # k > V
    assert f(P, 0, 4, 5000, 2049, P, P, None) == VL_EINVAL  # k > 2048
    assert f(P, 0, 4, 0, 1, P, P, None) == VL_EINVAL
    assert f(P, 0, -1, 10, 2, P, P, None) == VL_EINVAL
    assert f(P, 0, 1 << 31, 4, 2, P, P, None) == VL_EINVAL  # more rows than workgroups
    assert f(None, 0, 4, 10, 2, P, P, None) == VL_EINVAL
    assert f(P, 0, 4, 10, 2, None, P, None) == VL_EINVAL
    assert f(P, 0, 4, 10, 2, P, None, None) == VL_EINVAL
    assert f(None, 1, 0, 10, 2, None, None, None) == VL_OK


def test_slice_acc_host_checks(lib):
    f = lib.vl_slice_acc
    assert f(P, P, -1, None) == VL_EINVAL
    assert f(None, P, 4, None) == VL_EINVAL
    assert f(P, None, 4, None) == VL_EINVAL
    assert f(None, None, 0, None) == VL_OK


def test_head_scratch_bytes(lib):
    f = lib.vl_head_scratch_bytes
    a = 256
    up = lambda b: (b + a - 1) // a * a  # noqa: E731
    # logits, half hidden rows (hs padded to 64), half gradient, (max, sum)
    # records per 128 columns, lse, loss sums per 2048 columns, workspace
    want = (up(32 * 1024 * 4) + up(32 * 256 * 2) + up(32 * 1024 * 2) + up(32 * 8 * 8)
            + up(32 * 4) + up(32 * 1 * 4) + (64 << 20))
    assert f(32, 1024, 256) == want
    want = (up(5 * 1000 * 4) + up(5 * 128 * 2) + up(5 * 1000 * 2) + up(5 * 8 * 8)
            + up(5 * 4) + up(5 * 1 * 4) + (64 << 20))
    assert f(5, 1000, 72) == want
    assert f(0, 1024, 256) == 0 and f(32, 0, 256) == 0 and f(32, 1024, 0) == 0
    assert f(32, (1 << 19) + 1, 256) == 0


@pytest.mark.parametrize("name", ["vl_head_kl", "vl_head_kl_tune"])
def test_head_host_checks(lib, name):
    f = getattr(lib, name)
    ok = dict(x=P, w=P, wd=1, ids=P, probs=P, k=4, dx=P, loss=P, ntok=8, V=64, hs=16,
              total=8, gscale=1.0, chunk=4, scratch=P, sb=1 << 40, st=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["w"], a["wd"], a["ids"], a["probs"], a["k"], a["dx"], a["loss"],
                 a["ntok"], a["V"], a["hs"], a["total"], a["gscale"], a["chunk"], a["scratch"],
                 a["sb"], a["st"])
    assert call(wd=0) == VL_EDTYPE  # float32 weights are not a head type
    assert call(wd=3) == VL_EDTYPE
    assert call(k=0) == VL_EINVAL
    assert call(k=65) == VL_EINVAL
    assert call(V=(1 << 19) + 1) == VL_EINVAL
    assert call(hs=0) == VL_EINVAL
    assert call(total=0) == VL_EINVAL
    assert call(chunk=0) == VL_EINVAL
    assert call(gscale=0.0) == VL_EINVAL
    assert call(gscale=float("inf")) == VL_EINVAL
    assert call(gscale=float("nan")) == VL_EINVAL
    assert call(ntok=-1) == VL_EINVAL
    assert call(sb=1000) == VL_EINVAL  # scratch too small
    for name in ("x", "w", "ids", "probs", "dx", "loss", "scratch"):
        assert call(**{name: None}) == VL_EINVAL, name
    assert call(ntok=0, x=None, scratch=None) == VL_OK


P16 = ctypes.c_void_p(0x2000)  # 16-byte aligned, never dereferenced
P4 = ctypes.c_void_p(0x2004)   # 4-byte aligned only


def slice_fwd(lib, **kw):
    a = dict(logits=P, dtype=0, ld=16, off=0, width=16, ids=P, probs=P, k=2, part=P16,
             ntok=4, rng=None, stream=None)
    a.update(kw)
    return lib.vl_kl_slice_fwd(a["logits"], a["dtype"], a["ld"], a["off"], a["width"],
                               a["ids"], a["probs"], a["k"], a["part"], a["ntok"], a["rng"],
                               a["stream"])


def slice_bwd(lib, **kw):
    a = dict(logits=P, dtype=0, ld=16, off=0, width=16, ids=P, probs=P, k=2, lse=P,
             ntok=4, rng=None, coef=1.0, stream=None)
    a.update(kw)
    return lib.vl_kl_slice_bwd(a["logits"], a["dtype"], a["ld"], a["off"], a["width"],
                               a["ids"], a["probs"], a["k"], a["lse"], a["ntok"], a["rng"],
                               a["coef"], a["stream"])


def test_slice_host_checks(lib):
    for f in (slice_fwd, slice_bwd):
        assert f(lib, dtype=2) == VL_EDTYPE
        assert f(lib, width=0) == VL_EINVAL
        assert f(lib, ld=15) == VL_EINVAL  # rows would overlap
        assert f(lib, off=-1) == VL_EINVAL
        assert f(lib, off=(1 << 31) - 16) == VL_EINVAL  # off + width past 2^31 - 1
        assert f(lib, k=0) == VL_EINVAL
        assert f(lib, ntok=-1) == VL_EINVAL
        assert f(lib, ntok=1 << 62, ld=1 << 20, width=1 << 20) == VL_EINVAL
        assert f(lib, rng=rng(4, 3, 2)) == VL_EINVAL
        for name in ("logits", "ids", "probs"):
            assert f(lib, **{name: None}) == VL_EINVAL, name
        assert f(lib, ntok=0, logits=None, ids=None, probs=None) == VL_OK
    assert slice_fwd(lib, part=None) == VL_EINVAL
    assert slice_fwd(lib, part=P4) == VL_EINVAL  # parts are 16-byte records
    assert slice_bwd(lib, lse=None) == VL_EINVAL


def test_slice_merge_host_checks(lib):
    f = lib.vl_kl_slice_merge
    assert f(P16, 0, P, None, 4, None, None) == VL_EINVAL
    assert f(P16, 2, P, None, -1, None, None) == VL_EINVAL
    assert f(None, 2, P, None, 4, None, None) == VL_EINVAL
    assert f(P4, 2, P, None, 4, None, None) == VL_EINVAL
    assert f(P16, 2, None, None, 4, None, None) == VL_EINVAL
    assert f(P16, 2, P, None, 4, rng(0, 0, 0), None) == VL_EINVAL
    assert f(None, 2, None, None, 0, None, None) == VL_OK


def ce_ws(lib, **kw):
    a = dict(logits=P, dtype=0, labels=P, loss=P, lse=None, ntok=4, V=10, rng=None,
             scale=1.0, ws=P, ws_bytes=lib.vl_split_workspace_bytes(), stream=None)
    a.update(kw)
    return lib.vl_ce_fwd_bwd_ws(a["logits"], a["dtype"], a["labels"], a["loss"], a["lse"],
                                a["ntok"], a["V"], a["rng"], a["scale"], a["ws"],
                                a["ws_bytes"], a["stream"])


def kl_ws(lib, **kw):
    a = dict(logits=P, dtype=0, ids=P, probs=P, k=2, loss=P, lse=None, ntok=4, V=10,
             rng=None, coef=1.0, ws=P, ws_bytes=lib.vl_split_workspace_bytes(), stream=None)
    a.update(kw)
    return lib.vl_kl_fwd_bwd_ws(a["logits"], a["dtype"], a["ids"], a["probs"], a["k"],
                                a["loss"], a["lse"], a["ntok"], a["V"], a["rng"], a["coef"],
                                a["ws"], a["ws_bytes"], a["stream"])


def test_split_workspace_calls_host_checks(lib):
    n = lib.vl_split_workspace_bytes()
    assert n == 256 * 1024
    for f in (ce_ws, kl_ws):
        assert f(lib, dtype=2) == VL_EDTYPE
        assert f(lib, V=0) == VL_EINVAL
        assert f(lib, ntok=-1) == VL_EINVAL
        assert f(lib, rng=rng(0, 0, 0)) == VL_EINVAL
        assert f(lib, rng=rng(8, 5, 3)) == VL_EINVAL
        assert f(lib, ws=None) == VL_EINVAL
        assert f(lib, ws_bytes=n - 1) == VL_EINVAL
        assert f(lib, logits=None) == VL_EINVAL
        assert f(lib, loss=None) == VL_EINVAL
        assert f(lib, ntok=0, ws=None) == VL_OK  # no rows: nothing to check or run
    assert kl_ws(lib, k=0) == VL_EINVAL
    assert kl_ws(lib, k=11) == VL_EINVAL
    assert kl_ws(lib, V=(1 << 19) + 8, k=4) == VL_EINVAL
    assert kl_ws(lib, ids=None) == VL_EINVAL
    assert kl_ws(lib, probs=None) == VL_EINVAL
    assert ce_ws(lib, labels=None) == VL_EINVAL


def test_noalloc_host_checks(lib):
    def f(**kw):
        a = dict(logits=P, dtype=0, ids=P, probs=P, k=2, loss=P, lse=None, ntok=4, V=10,
                 rng=None, coef=1.0, stream=None)
        a.update(kw)
        return lib.vl_kl_fwd_bwd_noalloc(a["logits"], a["dtype"], a["ids"], a["probs"], a["k"],
                                         a["loss"], a["lse"], a["ntok"], a["V"], a["rng"],
                                         a["coef"], a["stream"])
    assert f(dtype=2) == VL_EDTYPE
    assert f(V=0) == VL_EINVAL
    assert f(k=0) == VL_EINVAL
    assert f(k=11) == VL_EINVAL
    assert f(V=(1 << 19) + 8, k=4) == VL_EINVAL
    assert f(ntok=-1) == VL_EINVAL
    assert f(rng=rng(8, 5, 3)) == VL_EINVAL
    for name in ("logits", "ids", "probs", "loss"):
        assert f(**{name: None}) == VL_EINVAL
    assert f(ntok=0, logits=None) == VL_OK


@pytest.mark.parametrize("call", ["vl_head_topk", "vl_head_topk_tune"])
def test_head_topk_host_checks(lib, call):
    fn = getattr(lib, call)
    n = lib.vl_head_topk_scratch_bytes(8, 1000, 64)
    assert n >= 8 * 1000 * 4 + 8 * 64 * 2 + (64 << 20)
    assert lib.vl_head_topk_scratch_bytes(0, 1000, 64) == 0
    assert lib.vl_head_topk_scratch_bytes(8, 0, 64) == 0

    def f(**kw):
        a = dict(x=P, w=P, wd=1, ntok=4, V=1000, hs=64, k=16, ids=P, probs=P, chunk=8,
                 scratch=P, sb=n, stream=None)
        a.update(kw)
        return fn(a["x"], a["w"], a["wd"], a["ntok"], a["V"], a["hs"], a["k"], a["ids"],
                  a["probs"], a["chunk"], a["scratch"], a["sb"], a["stream"])
    assert f(wd=0) == VL_EDTYPE
    assert f(k=0) == VL_EINVAL
    assert f(k=1001) == VL_EINVAL
    assert f(V=5000, k=2049) == VL_EINVAL
    assert f(hs=0) == VL_EINVAL
    assert f(chunk=0) == VL_EINVAL
    assert f(ntok=-1) == VL_EINVAL
    n4 = lib.vl_head_topk_scratch_bytes(4, 1000, 64)  # min(chunk, ntok) rows
    assert f(sb=n4 - 1) == VL_EINVAL
    for name in ("x", "w", "ids", "probs", "scratch"):
        assert f(**{name: None}) == VL_EINVAL
    assert f(ntok=0, x=None) == VL_OK

