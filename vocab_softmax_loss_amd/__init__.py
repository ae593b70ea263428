"""Python binding of libvl.so, the fused vocabulary-softmax loss for MI355X.

The functions carry the C ABI's names and arguments (include/vl.h).  They only
marshal arguments: check that tensors are contiguous device tensors of the
right dtype and shape, pass their device pointers and the current HIP stream,
and raise on a non-zero status.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  Importing this module fails
loudly when libvl.so has not been built.

Tensors:
  logits  [ntok][V] torch.float32 or torch.bfloat16 (in place for the losses)
  labels  [ntok], ids [ntok][k]: torch.int32 or torch.uint32 (read as uint32)
  probs   [ntok][k] torch.float32
  loss, lse [ntok] torch.float32
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "VL_F32", "VL_BF16", "VL_F16", "VLError", "lib_path",
    "vl_ce_fwd_bwd", "vl_ce_fwd", "vl_ce_bwd", "vl_loss_mean", "vl_kl_fwd_bwd",
    "vl_topk_renorm", "vl_slice_acc", "vl_head_scratch_bytes", "vl_head_kl",
    "vl_kl_slice_fwd", "vl_kl_slice_merge", "vl_kl_slice_bwd", "vl_strerror",
    "vl_split_workspace_bytes", "vl_ce_fwd_bwd_ws", "vl_kl_fwd_bwd_ws", "vl_kl_fwd_bwd_noalloc",
    "vl_head_topk_scratch_bytes", "vl_head_topk",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libvl.so")

VL_F32 = 0
VL_BF16 = 1
VL_F16 = 2


class VLError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {vl_strerror(status)} (status {status})")
        self.status = status


class vl_range(ctypes.Structure):
    _fields_ = [("seq_len", ctypes.c_int64), ("start", ctypes.c_int64),
                ("end", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python vocab_softmax_loss_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    rp = ctypes.POINTER(vl_range)
    lib.vl_ce_fwd_bwd.argtypes = [vp, i32, vp, vp, vp, i64, i64, rp, f32, vp]
    lib.vl_ce_fwd.argtypes = [vp, i32, vp, vp, vp, i64, i64, rp, vp]
    lib.vl_ce_bwd.argtypes = [vp, i32, vp, vp, i64, i64, rp, f32, vp]
    lib.vl_loss_mean.argtypes = [vp, i64, rp, vp, vp]
    lib.vl_kl_fwd_bwd.argtypes = [vp, i32, vp, vp, i64, vp, vp, i64, i64, rp, f32, vp]
    lib.vl_topk_renorm.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    lib.vl_slice_acc.argtypes = [vp, vp, i64, vp]
    lib.vl_head_scratch_bytes.argtypes = [i64, i64, i64]
    lib.vl_head_scratch_bytes.restype = ctypes.c_size_t
    lib.vl_head_kl.argtypes = [vp, vp, i32, vp, vp, i64, vp, vp, i64, i64, i64, i64, f32, i64,
                               vp, ctypes.c_size_t, vp]
    lib.vl_head_kl.restype = i32
    lib.vl_head_kl_tune.argtypes = lib.vl_head_kl.argtypes
    lib.vl_head_kl_tune.restype = i32
    lib.vl_kl_slice_fwd.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, vp, i64, rp, vp]
    lib.vl_kl_slice_merge.argtypes = [vp, i64, vp, vp, i64, rp, vp]
    lib.vl_kl_slice_bwd.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, vp, i64, rp, f32, vp]
    sz = ctypes.c_size_t
    lib.vl_split_workspace_bytes.argtypes = []
    lib.vl_split_workspace_bytes.restype = sz
    lib.vl_ce_fwd_bwd_ws.argtypes = [vp, i32, vp, vp, vp, i64, i64, rp, f32, vp, sz, vp]
    lib.vl_kl_fwd_bwd_ws.argtypes = [vp, i32, vp, vp, i64, vp, vp, i64, i64, rp, f32, vp, sz,
                                     vp]
    lib.vl_kl_fwd_bwd_noalloc.argtypes = [vp, i32, vp, vp, i64, vp, vp, i64, i64, rp, f32, vp]
    lib.vl_head_topk_scratch_bytes.argtypes = [i64, i64, i64]
    lib.vl_head_topk_scratch_bytes.restype = sz
    lib.vl_head_topk.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, i64, vp, sz, vp]
    lib.vl_head_topk.restype = i32
    lib.vl_head_topk_tune.argtypes = lib.vl_head_topk.argtypes
    lib.vl_head_topk_tune.restype = i32
    lib.vl_strerror.argtypes = [i32]
    lib.vl_strerror.restype = ctypes.c_char_p
    for f in (lib.vl_ce_fwd_bwd, lib.vl_ce_fwd, lib.vl_ce_bwd, lib.vl_loss_mean,
              lib.vl_kl_fwd_bwd, lib.vl_topk_renorm, lib.vl_slice_acc, lib.vl_kl_slice_fwd,
              lib.vl_kl_slice_merge, lib.vl_kl_slice_bwd, lib.vl_ce_fwd_bwd_ws,
              lib.vl_kl_fwd_bwd_ws, lib.vl_kl_fwd_bwd_noalloc):
        f.restype = i32
    return lib


_lib = _load()


def lib_path() -> str:
    return _LIB_PATH


def vl_strerror(status: int) -> str:
    return _lib.vl_strerror(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return VL_F32
    if t.dtype == torch.bfloat16:
        return VL_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtypes, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


_INT_IDS = (torch.int32, torch.uint32)


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream)


def _range(rng):
    if rng is None:
        return None
    r = vl_range(*[int(v) for v in rng])
    return ctypes.byref(r)


def _check(status: int, where: str):
    if status != 0:
        raise VLError(status, where)


def vl_ce_fwd_bwd(logits, labels, loss, lse=None, rng=None, scale=1.0, stream=None):
    """Fused CE forward + in-place backward; see vl_ce_fwd_bwd in vl.h.
    ``rng`` is (seq_len, start, end) or None."""
    ntok, V = logits.shape
    with torch.cuda.device(logits.device):
        _check(_lib.vl_ce_fwd_bwd(
            _dev(logits, "logits", None), _dtype_code(logits),
            _dev(labels, "labels", _INT_IDS, (ntok,)),
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            None if lse is None else _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, V, _range(rng), float(scale), _stream(logits, stream)), "vl_ce_fwd_bwd")


def vl_ce_fwd(logits, labels, loss, lse=None, rng=None, stream=None):
    """CE forward only (logits read only); see vl_ce_fwd in vl.h."""
    ntok, V = logits.shape
    with torch.cuda.device(logits.device):
        _check(_lib.vl_ce_fwd(
            _dev(logits, "logits", None), _dtype_code(logits),
            _dev(labels, "labels", _INT_IDS, (ntok,)),
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            None if lse is None else _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, V, _range(rng), _stream(logits, stream)), "vl_ce_fwd")


def vl_ce_bwd(logits, labels, lse, rng=None, scale=1.0, stream=None):
    """CE backward from a saved lse, written over the logits; see vl_ce_bwd."""
    ntok, V = logits.shape
    with torch.cuda.device(logits.device):
        _check(_lib.vl_ce_bwd(
            _dev(logits, "logits", None), _dtype_code(logits),
            _dev(labels, "labels", _INT_IDS, (ntok,)),
            _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, V, _range(rng), float(scale), _stream(logits, stream)), "vl_ce_bwd")


def vl_loss_mean(loss, mean, rng=None, stream=None):
    """mean[0] = loss.sum() / (rows in rng), on the device; see vl_loss_mean."""
    ntok = loss.numel()
    with torch.cuda.device(loss.device):
        _check(_lib.vl_loss_mean(
            _dev(loss, "loss", (torch.float32,), (ntok,)), ntok, _range(rng),
            _dev(mean, "mean", (torch.float32,), (1,)), _stream(loss, stream)), "vl_loss_mean")


def vl_kl_fwd_bwd(logits, ids, probs, loss, lse=None, rng=None, coef=1.0, stream=None):
    """Fused distillation KL forward + in-place backward; see vl_kl_fwd_bwd."""
    ntok, V = logits.shape
    k = ids.shape[1] if ids.dim() == 2 else 0
    with torch.cuda.device(logits.device):
        _check(_lib.vl_kl_fwd_bwd(
            _dev(logits, "logits", None), _dtype_code(logits),
            _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)), k,
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            None if lse is None else _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, V, _range(rng), float(coef), _stream(logits, stream)), "vl_kl_fwd_bwd")


def vl_split_workspace_bytes():
    """Bytes of workspace the *_ws calls need at least."""
    return int(_lib.vl_split_workspace_bytes())


def _ws(workspace):
    return _dev(workspace, "workspace", (torch.uint8,)), workspace.numel()


def vl_ce_fwd_bwd_ws(logits, labels, loss, workspace, lse=None, rng=None, scale=1.0,
                     stream=None):
    """vl_ce_fwd_bwd with a workspace (a uint8 device tensor of at least
    vl_split_workspace_bytes() bytes) for rows split over several
    workgroups; see vl_ce_fwd_bwd_ws in vl.h."""
    ntok, V = logits.shape
    wp, wn = _ws(workspace)
    with torch.cuda.device(logits.device):
        _check(_lib.vl_ce_fwd_bwd_ws(
            _dev(logits, "logits", None), _dtype_code(logits),
            _dev(labels, "labels", _INT_IDS, (ntok,)),
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            None if lse is None else _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, V, _range(rng), float(scale), wp, wn, _stream(logits, stream)),
            "vl_ce_fwd_bwd_ws")


def vl_kl_fwd_bwd_ws(logits, ids, probs, loss, workspace, lse=None, rng=None, coef=1.0,
                     stream=None):
    """vl_kl_fwd_bwd with a workspace for rows split over several
    workgroups; see vl_kl_fwd_bwd_ws in vl.h."""
    ntok, V = logits.shape
    k = ids.shape[1] if ids.dim() == 2 else 0
    wp, wn = _ws(workspace)
    with torch.cuda.device(logits.device):
        _check(_lib.vl_kl_fwd_bwd_ws(
            _dev(logits, "logits", None), _dtype_code(logits),
            _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)), k,
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            None if lse is None else _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, V, _range(rng), float(coef), wp, wn, _stream(logits, stream)),
            "vl_kl_fwd_bwd_ws")


def vl_kl_fwd_bwd_noalloc(logits, ids, probs, loss, lse=None, rng=None, coef=1.0, stream=None):
    """vl_kl_fwd_bwd_ws with the library's own device mailbox in place of a
    workspace (nothing is allocated); see vl_kl_fwd_bwd_noalloc in vl.h."""
    ntok, V = logits.shape
    k = ids.shape[1] if ids.dim() == 2 else 0
    with torch.cuda.device(logits.device):
        _check(_lib.vl_kl_fwd_bwd_noalloc(
            _dev(logits, "logits", None), _dtype_code(logits),
            _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)), k,
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            None if lse is None else _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, V, _range(rng), float(coef), _stream(logits, stream)),
            "vl_kl_fwd_bwd_noalloc")


def vl_topk_renorm(logits, k, ids, probs, stream=None):
    """Teacher top-k ids and renormalised probabilities; see vl_topk_renorm."""
    ntok, V = logits.shape
    with torch.cuda.device(logits.device):
        _check(_lib.vl_topk_renorm(
            _dev(logits, "logits", None), _dtype_code(logits), ntok, V, int(k),
            _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)),
            _stream(logits, stream)), "vl_topk_renorm")


def vl_slice_acc(dst, src, stream=None):
    """dst += src (float32, bit-exact); see vl_slice_acc."""
    n = dst.numel()
    with torch.cuda.device(dst.device):
        _check(_lib.vl_slice_acc(
            _dev(dst, "dst", (torch.float32,)),
            _dev(src, "src", (torch.float32,), tuple(dst.shape)), n,
            _stream(dst, stream)), "vl_slice_acc")


def vl_head_scratch_bytes(chunk, V, hs):
    """Bytes of scratch vl_head_kl needs for `chunk` rows at a time."""
    return int(_lib.vl_head_scratch_bytes(int(chunk), int(V), int(hs)))


def vl_head_kl(x, w, ids, probs, dx, loss, total, gscale, chunk, scratch, stream=None,
               tune=False):
    """Vocabulary head + distillation KL; see vl_head_kl in vl.h.  ``w`` is
    a torch.float16 or torch.bfloat16 [V][hs] tensor; ``scratch`` a uint8
    device tensor of at least vl_head_scratch_bytes(min(chunk, ntok), V, hs)
    bytes.  ``tune=True`` calls vl_head_kl_tune instead (times hipBLASLt's
    candidates for shapes not yet tuned; the host waits)."""
    ntok, hs = x.shape
    V = w.shape[0]
    k = ids.shape[1] if ids.dim() == 2 else 0
    wd = {torch.float16: VL_F16, torch.bfloat16: VL_BF16}.get(w.dtype)
    if wd is None:
        raise TypeError(f"w must be float16 or bfloat16, got {w.dtype}")
    with torch.cuda.device(x.device):
        fn, name = (_lib.vl_head_kl_tune, "vl_head_kl_tune") if tune else (_lib.vl_head_kl,
                                                                            "vl_head_kl")
        _check(fn(
            _dev(x, "x", (torch.float32,)), _dev(w, "w", None, (V, hs)), wd,
            _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)), k,
            _dev(dx, "dx", (torch.float32,), (ntok, hs)),
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            ntok, V, hs, int(total), float(gscale), int(chunk),
            _dev(scratch, "scratch", (torch.uint8,)), scratch.numel(),
            _stream(x, stream)), name)


def vl_head_topk_scratch_bytes(chunk, V, hs):
    """Bytes of scratch vl_head_topk needs for `chunk` rows at a time."""
    return int(_lib.vl_head_topk_scratch_bytes(int(chunk), int(V), int(hs)))


def vl_head_topk(x, w, k, ids, probs, chunk, scratch, stream=None, tune=False):
    """Teacher-side vocabulary head: top-k ids and renormalised
    probabilities of half(x) . w^T; see vl_head_topk in vl.h.  ``w`` is a
    torch.float16 or torch.bfloat16 [V][hs] tensor; ``scratch`` a uint8
    device tensor of at least vl_head_topk_scratch_bytes(min(chunk, ntok),
    V, hs) bytes.  ``tune=True`` calls vl_head_topk_tune instead."""
    ntok, hs = x.shape
    V = w.shape[0]
    wd = {torch.float16: VL_F16, torch.bfloat16: VL_BF16}.get(w.dtype)
    if wd is None:
        raise TypeError(f"w must be float16 or bfloat16, got {w.dtype}")
    with torch.cuda.device(x.device):
        fn, name = ((_lib.vl_head_topk_tune, "vl_head_topk_tune") if tune
                    else (_lib.vl_head_topk, "vl_head_topk"))
        _check(fn(
            _dev(x, "x", (torch.float32,)), _dev(w, "w", None, (V, hs)), wd, ntok, V, hs,
            int(k), _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)), int(chunk),
            _dev(scratch, "scratch", (torch.uint8,)), scratch.numel(),
            _stream(x, stream)), name)


def _slice_rows(t: torch.Tensor, name: str):
    """Pointer and row stride of a [ntok][width] slice whose rows may be a
    column window of a wider buffer (element stride 1, row stride >= width)."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    ntok, width = t.shape
    if width > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    ld = t.stride(0) if ntok > 1 else width
    if ld < width:
        raise ValueError(f"{name} rows overlap (row stride {ld} < width {width})")
    return t.data_ptr(), int(ld)


def vl_kl_slice_fwd(logits, off, ids, probs, part, rng=None, stream=None):
    """Statistics (a, z, P, w) of one vocabulary slice; see vl_kl_slice_fwd.
    ``logits`` [ntok][width] holds vocabulary ids [off, off + width); it may
    be a column window of a wider tensor.  ``part`` is a [ntok][4]
    float32 tensor."""
    ntok, width = logits.shape
    k = ids.shape[1] if ids.dim() == 2 else 0
    ptr, ld = _slice_rows(logits, "logits")
    with torch.cuda.device(logits.device):
        _check(_lib.vl_kl_slice_fwd(
            ptr, _dtype_code(logits), ld, int(off), width,
            _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)), k,
            _dev(part, "part", (torch.float32,), (ntok, 4)),
            ntok, _range(rng), _stream(logits, stream)), "vl_kl_slice_fwd")


def vl_kl_slice_merge(parts, loss, lse=None, rng=None, stream=None):
    """Whole-row loss and lse from every slice's part ([nslice][ntok][4]
    float32); see vl_kl_slice_merge."""
    nslice, ntok = parts.shape[0], parts.shape[1]
    with torch.cuda.device(parts.device):
        _check(_lib.vl_kl_slice_merge(
            _dev(parts, "parts", (torch.float32,), (nslice, ntok, 4)), nslice,
            _dev(loss, "loss", (torch.float32,), (ntok,)),
            None if lse is None else _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, _range(rng), _stream(parts, stream)), "vl_kl_slice_merge")


def vl_kl_slice_bwd(logits, off, ids, probs, lse, rng=None, coef=1.0, stream=None):
    """Gradient of one vocabulary slice from the merged lse, written over
    the slice; see vl_kl_slice_bwd."""
    ntok, width = logits.shape
    k = ids.shape[1] if ids.dim() == 2 else 0
    ptr, ld = _slice_rows(logits, "logits")
    with torch.cuda.device(logits.device):
        _check(_lib.vl_kl_slice_bwd(
            ptr, _dtype_code(logits), ld, int(off), width,
            _dev(ids, "ids", _INT_IDS, (ntok, k)),
            _dev(probs, "probs", (torch.float32,), (ntok, k)), k,
            _dev(lse, "lse", (torch.float32,), (ntok,)),
            ntok, _range(rng), float(coef), _stream(logits, stream)), "vl_kl_slice_bwd")
