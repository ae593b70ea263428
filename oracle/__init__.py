"""Float64 CPU oracle of the fused vocabulary-softmax loss (ctypes loader).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.  The row
arithmetic is in ``oracle.c``; this module builds that file with gcc, loads
it and marshals numpy arrays.  The vocabulary head (``head_kl``) is numpy
float64 here: two library matrix products around the KL rows.

Logits are numpy arrays ``[n][V]``: float32, or uint16 holding bf16 bit
patterns.  Labels and ids are read as uint32.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_c_double_p = ctypes.POINTER(ctypes.c_double)
_c_i64_p = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            vp, i64, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
            lib.oracle_row_lse.argtypes = [vp, ctypes.c_int, i64]
            lib.oracle_row_lse.restype = dbl
            lib.oracle_ce.argtypes = [vp, ctypes.c_int, vp, i64, i64, vp, i64, i64,
                                      i64, dbl, vp, vp, vp]
            lib.oracle_ce.restype = None
            lib.oracle_ce_bwd.argtypes = [vp, ctypes.c_int, vp, vp, i64, i64, vp, i64, i64,
                                          i64, dbl, vp]
            lib.oracle_ce_bwd.restype = None
            lib.oracle_loss_mean.argtypes = [vp, i64, i64, i64, i64]
            lib.oracle_loss_mean.restype = dbl
            lib.oracle_kl.argtypes = [vp, ctypes.c_int, vp, vp, i64, i64, i64, vp,
                                      i64, i64, i64, dbl, vp, vp, vp]
            lib.oracle_kl.restype = None
            lib.oracle_topk.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp]
            lib.oracle_topk.restype = None
            lib.oracle_acc.argtypes = [vp, vp, i64, vp]
            lib.oracle_acc.restype = None
            lib.oracle_threads.argtypes = []
            lib.oracle_threads.restype = ctypes.c_int
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_threads.restype = None
            _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows2d(logits: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(logits)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    return a


def _range_args(rng):
    if rng is None:
        return 0, 0, 0
    seq_len, start, end = rng
    return int(seq_len), int(start), int(end)


def threads() -> int:
    """Host threads the oracle's row loops use (the OpenMP runtime's
    current maximum)."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Use n >= 1 host threads from now on (timing only; no arithmetic
    changes)."""
    _load().oracle_set_threads(int(n))


def row_lse(row: np.ndarray) -> float:
    a = np.ascontiguousarray(row).reshape(-1)
    return _load().oracle_row_lse(_ptr(a), _dtype_code(a), a.size)


def ce(logits, labels, rng=None, scale=1.0, row_index=None, want_grad=True):
    """Per-row loss, lse and (optionally) the scaled gradient, all float64."""
    a = _rows2d(logits)
    n, V = a.shape
    lab = np.ascontiguousarray(labels).astype(np.uint32, copy=False).reshape(-1)
    assert lab.size == n
    ridx = None if row_index is None else np.ascontiguousarray(row_index, dtype=np.int64)
    loss = np.empty(n)
    lse = np.empty(n)
    grad = np.empty((n, V)) if want_grad else None
    sl, st, en = _range_args(rng)
    _load().oracle_ce(_ptr(a), _dtype_code(a), _ptr(lab), n, V, _ptr(ridx), sl, st, en,
                      float(scale), _ptr(loss), _ptr(lse), _ptr(grad))
    return loss, lse, grad


def ce_bwd(logits, labels, lse, rng=None, scale=1.0, row_index=None):
    """float64 gradient from a saved float32 logsumexp per row."""
    a = _rows2d(logits)
    n, V = a.shape
    lab = np.ascontiguousarray(labels).astype(np.uint32, copy=False).reshape(-1)
    L = np.ascontiguousarray(lse, dtype=np.float32).reshape(-1)
    assert lab.size == n and L.size == n
    ridx = None if row_index is None else np.ascontiguousarray(row_index, dtype=np.int64)
    grad = np.empty((n, V))
    sl, st, en = _range_args(rng)
    _load().oracle_ce_bwd(_ptr(a), _dtype_code(a), _ptr(lab), _ptr(L), n, V, _ptr(ridx), sl,
                          st, en, float(scale), _ptr(grad))
    return grad


def loss_mean(loss, rng=None):
    """Mean of a float32 loss vector over the loss range, as float64."""
    x = np.ascontiguousarray(loss, dtype=np.float32).reshape(-1)
    sl, st, en = _range_args(rng)
    return _load().oracle_loss_mean(_ptr(x), x.size, sl, st, en)


def kl(logits, ids, probs, rng=None, coef=1.0, row_index=None, want_grad=True):
    """Per-row KL, lse and (optionally) the scaled gradient, all float64."""
    a = _rows2d(logits)
    n, V = a.shape
    idv = np.ascontiguousarray(ids).astype(np.uint32, copy=False).reshape(n, -1)
    k = idv.shape[1]
    pv = np.ascontiguousarray(probs, dtype=np.float32).reshape(n, k)
    ridx = None if row_index is None else np.ascontiguousarray(row_index, dtype=np.int64)
    loss = np.empty(n)
    lse = np.empty(n)
    grad = np.empty((n, V)) if want_grad else None
    sl, st, en = _range_args(rng)
    _load().oracle_kl(_ptr(a), _dtype_code(a), _ptr(idv), _ptr(pv), k, n, V, _ptr(ridx),
                      sl, st, en, float(coef), _ptr(loss), _ptr(lse), _ptr(grad))
    return loss, lse, grad


def topk(logits, k):
    """ids (uint32, [n][k], in output order) and float64 probs."""
    a = _rows2d(logits)
    n, V = a.shape
    ids = np.empty((n, k), dtype=np.uint32)
    probs = np.empty((n, k))
    _load().oracle_topk(_ptr(a), _dtype_code(a), n, V, int(k), _ptr(ids), _ptr(probs))
    return ids, probs


def acc(dst, src):
    """float32 dst + src, element-wise."""
    d = np.ascontiguousarray(dst, dtype=np.float32).reshape(-1)
    s = np.ascontiguousarray(src, dtype=np.float32).reshape(-1)
    assert d.size == s.size
    out = np.empty_like(d)
    _load().oracle_acc(_ptr(d), _ptr(s), d.size, _ptr(out))
    return out.reshape(np.shape(dst))


# ---------------------------------------------------------------- head

def round_half(x, dtype):
    """float32 values rounded to nearest even in "f16" or "bf16", returned
    as float64.  The hidden rows and the head weights are rounded once
    this way before both products."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return f.astype(np.float16).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def head_kl(x, w, ids, probs, total, gscale):
    """Vocabulary head with the distillation KL (cortiq-engine
    train_head.rs, head_kl), float64, on hidden rows ``x`` [n][hs] and head
    ``w`` [V][hs] given as float64 values (already rounded the way the GPU
    rounds them, see ``round_half``):

      s_t = w x_t                                  (logits, a library matmul)
      loss_t = sum over q with p_q > 0 of p_q (ln p_q - (s_t[id_q] - lse_t))
      d_t = (gscale / total) (softmax(s_t) - t_t)  (the KL rows' in-place gradient)
      dx_t = d_t w / gscale                        (the input gradient)

    so dx is the gradient of sum_t loss_t / total with the teacher term
    applied as given.  Returns (loss [n], dx [n][hs]), float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n = x.shape[0]
    idv = np.ascontiguousarray(ids).astype(np.int64).reshape(n, -1)
    pv = np.ascontiguousarray(probs, dtype=np.float32).astype(np.float64).reshape(n, -1)
    s = x @ w.T
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    loss = np.zeros(n)
    coef = float(gscale) / float(total)
    d = np.exp(s - lse[:, None])
    for t in range(n):
        for q in range(idv.shape[1]):
            pq = pv[t, q]
            if pq > 0.0:
                loss[t] += pq * (np.log(pq) - (s[t, idv[t, q]] - lse[t]))
            d[t, idv[t, q]] -= pq
    d *= coef
    dx = (d @ w) / float(gscale)
    return loss, dx


# ---------------------------------------------------- vocabulary slices

def head_topk(x, w, k):
    """The teacher side of the vocabulary head (cortiq-engine train_head.rs,
    host fn topk), float64, on hidden rows ``x`` [n][hs] and head ``w``
    [V][hs] given as float64 values (already rounded the way the GPU rounds
    them, see ``round_half``):

      s_t = w x_t                         (logits, a library matmul)
      ids_t = the k ids first in the order (s_t desc, id asc)
      probs_t[q] = exp(s_t[ids_q] - s_t[ids_0]) / sum_{q' < k} exp(...)

    The order is a stable library sort on (-s, id) of every column, ties to
    the lower id (-0 and +0 tie).  Returns (ids uint32 [n][k], probs float64
    [n][k]).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    s = x @ w.T
    n, V = s.shape
    k = int(k)
    ids = np.empty((n, k), dtype=np.uint32)
    probs = np.empty((n, k))
    cols = np.arange(V)
    for t in range(n):
        order = np.lexsort((cols, -s[t]))[:k]
        ids[t] = order
        v = s[t, order]
        e = np.exp(v - v[0])
        probs[t] = e / e.sum()
    return ids, probs


def _widen(logits) -> np.ndarray:
    """[n][w] float32 or bf16 bit patterns (uint16) as exact float64."""
    a = _rows2d(logits)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype != np.float32:
        raise TypeError(f"oracle logits must be float32 or uint16 (bf16 bits), got {a.dtype}")
    return a.astype(np.float64)


def _in_range(n, rng):
    if rng is None:
        return np.ones(n, dtype=bool)
    seq_len, start, end = rng
    pos = np.arange(n) % int(seq_len)
    return (pos >= int(start)) & (pos < int(end))


def kl_slice_part(slice_logits, off, ids, probs, rng=None):
    """Partial statistics of one vocabulary slice for the distillation KL
    (cortiq-engine train_head.rs: the module doc's loss, and the head's
    vocabulary cuts, each a column offset and a width).  The slice holds
    columns [off, off + width) of each row; per row, in float64:

      a = max of the slice's values (0 if it has no finite value)
      z = sum_j exp(s_j - a)
      P = sum of p_q over the teacher entries with off <= id_q < off + width
          and p_q > 0
      w = sum over the same entries of p_q (ln p_q - (s[id_q - off] - a))

    Rows outside the loss range get (0, 0, 0, 0).  Returns [n][4].
    """
    s = _widen(slice_logits)
    n, width = s.shape
    idv = np.ascontiguousarray(ids).astype(np.int64).reshape(n, -1)
    pv = np.ascontiguousarray(probs, dtype=np.float32).astype(np.float64).reshape(n, -1)
    live = _in_range(n, rng)
    out = np.zeros((n, 4))
    for t in range(n):
        if not live[t]:
            continue
        row = s[t]
        fin = row[np.isfinite(row)]
        a = float(fin.max()) if fin.size else 0.0
        z = float(np.exp(row - a).sum())
        P = 0.0
        w = 0.0
        for q in range(idv.shape[1]):
            j, p = idv[t, q] - off, pv[t, q]
            if 0 <= j < width and p > 0.0:
                P += p
                w += p * (math.log(p) - (row[j] - a))
        out[t] = (a, z, P, w)
    return out


def kl_slice_merge(parts, rng=None):
    """Loss and logsumexp of whole rows from the partial statistics of every
    slice of the vocabulary (``parts`` [S][n][4], as ``kl_slice_part``
    gives them), float64:

      lse  = ln sum_i z_i e^{a_i}      over the slices with z_i > 0
      loss = sum_i (w_i + P_i (lse - a_i))   over the slices with P_i > 0

    which is sum_q p_q (ln p_q - s_{id_q} + lse), the KL of the whole row,
    because the slices partition the vocabulary.  Rows outside the loss range
    get loss 0 and lse 0.  Returns (loss [n], lse [n]).
    """
    pa = np.asarray(parts, dtype=np.float64)
    S, n, _ = pa.shape
    live = _in_range(n, rng)
    loss = np.zeros(n)
    lse = np.zeros(n)
    for t in range(n):
        if not live[t]:
            continue
        a, z, P, w = pa[:, t, 0], pa[:, t, 1], pa[:, t, 2], pa[:, t, 3]
        has = z > 0.0
        M = float(a[has].max())
        L = M + math.log(float((z[has] * np.exp(a[has] - M)).sum()))
        lse[t] = L
        tgt = P > 0.0
        loss[t] = float((w[tgt] + P[tgt] * (L - a[tgt])).sum())
    return loss, lse


def kl_slice_bwd(slice_logits, off, ids, probs, lse, coef=1.0, rng=None):
    """Gradient of one vocabulary slice from the rows' logsumexp, used as
    given: g_j = coef (exp(s_j - lse) - t_j), t_j = p_q where id_q = off + j
    (else 0), the module doc's p_S - p_T restricted to the slice.  Rows
    outside the loss range get 0.  Returns [n][width] float64."""
    s = _widen(slice_logits)
    n, width = s.shape
    idv = np.ascontiguousarray(ids).astype(np.int64).reshape(n, -1)
    pv = np.ascontiguousarray(probs, dtype=np.float32).astype(np.float64).reshape(n, -1)
    L = np.asarray(lse, dtype=np.float64).reshape(-1)
    live = _in_range(n, rng)
    g = np.zeros((n, width))
    for t in range(n):
        if not live[t]:
            continue
        d = np.exp(s[t] - L[t])
        for q in range(idv.shape[1]):
            j = idv[t, q] - off
            if 0 <= j < width:
                d[j] -= pv[t, q]
        g[t] = float(coef) * d
    return g
