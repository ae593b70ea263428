"""Seeded synthetic inputs for the fused vocabulary-softmax loss.

This module draws random numbers and lays them out; it holds none of the
loss arithmetic.  Both the HIP path and the float64 oracle read the bytes it
produces (the oracle reads them after a copy to the host), so neither side
generates its own inputs.

Every recipe takes a ``seed`` and a ``device``.  Draws come from a
``torch.Generator`` on that device, so the same call on a CPU and on a GPU
gives different (but each reproducible) bytes; the checks never depend on
the particular values, only on both sides seeing the same ones.

The workloads stand in for language-model head logits; no dataset or trained
weights are involved.  The page-test recipes at the bottom take the shapes of
the two tests printed on the pages: the cross-entropy test's inputs as that
page states them, the KL test's shapes filled with this module's own seeded
draws.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# Row chunk used when drawing big tensors, to bound temporaries.
_CHUNK_ELEMS = 1 << 28


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _row_chunks(ntok: int, V: int):
    step = max(1, _CHUNK_ELEMS // max(V, 1))
    for r0 in range(0, ntok, step):
        yield r0, min(ntok, r0 + step)


def normal_logits(ntok: int, V: int, sigma: float, seed: int, device,
                  dtype=torch.float32) -> torch.Tensor:
    """``[ntok][V]`` logits ~ N(0, sigma^2); bf16 is the round-to-nearest-even
    cast of the float32 draw."""
    g = _gen(seed, device)
    out = torch.empty((ntok, V), dtype=dtype, device=device)
    for r0, r1 in _row_chunks(ntok, V):
        x = torch.randn((r1 - r0, V), generator=g, device=device, dtype=torch.float32)
        x.mul_(sigma)
        out[r0:r1].copy_(x)
    return out


def uniform_labels(ntok: int, V: int, seed: int, device) -> torch.Tensor:
    """``[ntok]`` labels uniform in [0, V), int32 (the ABI reads them as u32)."""
    g = _gen(seed, device)
    return torch.randint(0, V, (ntok,), generator=g, device=device, dtype=torch.int32)


def boost_label_rows(logits: torch.Tensor, labels: torch.Tensor, frac: float,
                     boost: float, seed: int) -> torch.Tensor:
    """Add ``boost`` to the label logit of exactly round(frac * ntok) rows,
    chosen by a seeded permutation (float32 add before upload).  Returns the
    chosen row indices."""
    ntok = logits.shape[0]
    nb = int(round(frac * ntok))
    g = _gen(seed, logits.device)
    rows = torch.randperm(ntok, generator=g, device=logits.device)[:nb]
    cols = labels[rows].long()
    logits[rows, cols] = logits[rows, cols] + boost
    return rows


def distinct_ids(ntok: int, V: int, k: int, seed: int, device) -> torch.Tensor:
    """``[ntok][k]`` int32 ids, distinct within each row, uniform over the
    k-subsets of [0, V), in random order."""
    g = _gen(seed, device)
    out = torch.empty((ntok, k), dtype=torch.int32, device=device)
    for r0, r1 in _row_chunks(ntok, V):
        u = torch.rand((r1 - r0, V), generator=g, device=device)
        out[r0:r1] = u.topk(k, dim=1).indices.to(torch.int32)
    return out


def softmax_probs(ntok: int, k: int, sigma: float, seed: int, device) -> torch.Tensor:
    """``[ntok][k]`` float32 teacher probabilities: the normalised exponential
    of N(0, sigma^2) draws, formed in float64 and cast once to float32."""
    g = _gen(seed, device)
    z = torch.randn((ntok, k), generator=g, device=device, dtype=torch.float64) * sigma
    z = z - z.max(dim=1, keepdim=True).values
    e = torch.exp(z)
    return (e / e.sum(dim=1, keepdim=True)).to(torch.float32)


def zipf_teacher(ntok: int, V: int, s: float, noise_sigma: float, seed: int,
                 device, shared_perm: bool = False) -> torch.Tensor:
    """``[ntok][V]`` float32 teacher logits ``2*ln(w_rank(id)) + N(0, noise^2)``
    with Zipf weights ``w_r = r^-s / H`` over ranks 1..V.  Ranks map to ids by
    one seeded permutation per row (or one shared by all rows)."""
    g = _gen(seed, device)
    r = torch.arange(1, V + 1, device=device, dtype=torch.float64)
    w = r.pow(-s)
    base = (2.0 * torch.log(w / w.sum())).to(torch.float32)
    out = torch.empty((ntok, V), dtype=torch.float32, device=device)
    shared = None
    if shared_perm:
        shared = torch.rand((1, V), generator=g, device=device).argsort(dim=1)
    for r0, r1 in _row_chunks(ntok, V):
        n = r1 - r0
        if shared is None:
            perm = torch.rand((n, V), generator=g, device=device).argsort(dim=1)
        else:
            perm = shared.expand(n, V)
        vals = base.unsqueeze(0) + noise_sigma * torch.randn(
            (n, V), generator=g, device=device, dtype=torch.float32)
        out[r0:r1].scatter_(1, perm, vals)
    return out


# ---------------------------------------------------------------------------
# Named workloads.  Sizes and distributions follow the five configurations of
# the benchmark specification; the names say what each one is.

@dataclass(frozen=True)
class Workload:
    name: str
    ntok: int
    V: int
    k: int = 0
    dtype: str = "f32"


CE_TINY = Workload("ce_64x512_f32", 64, 512)
CE_LM = Workload("ce_4096x32000_f32_prompt_masked", 4096, 32000)
TOPK_ZIPF = Workload("topk_4096x32000_f32_k64_zipf", 4096, 32000, 64)
KL_LARGE = Workload("kl_8192x128256_f32_k128", 8192, 128256, 128)
KL_BF16 = Workload("kl_16384x151936_bf16_k256_sliced", 16384, 151936, 256, "bf16")


def ce_tiny(device, seed: int = 1, ntok: int = 64, V: int = 512):
    """CE, tiny: logits ~ N(0, 2^2), labels uniform, every row in the loss,
    gradient scale 1/ntok."""
    logits = normal_logits(ntok, V, 2.0, seed * 1000 + 1, device)
    labels = uniform_labels(ntok, V, seed * 1000 + 2, device)
    return dict(logits=logits, labels=labels, rng=None, scale=1.0 / ntok)


def ce_lm(device, seed: int = 2, nseq: int = 8, seq_len: int = 512, V: int = 32000,
          prompt: int = 128):
    """CE at language-model shape: ``nseq`` sequences of ``seq_len`` tokens,
    logits ~ N(0, 3^2) with +6 at the label on 30% of rows, labels uniform,
    the first ``prompt`` tokens of each sequence outside the loss, scale =
    1 / (tokens in the loss)."""
    ntok = nseq * seq_len
    logits = normal_logits(ntok, V, 3.0, seed * 1000 + 1, device)
    labels = uniform_labels(ntok, V, seed * 1000 + 2, device)
    boost_label_rows(logits, labels, 0.3, 6.0, seed * 1000 + 3)
    rng = (seq_len, prompt, seq_len)
    n_in = nseq * (seq_len - prompt)
    return dict(logits=logits, labels=labels, rng=rng, scale=1.0 / n_in)


def topk_zipf(device, seed: int = 3, ntok: int = 4096, V: int = 32000, k: int = 64,
              shared_perm: bool = False):
    """Teacher top-k: Zipf(s=1.1) log-weights over a seeded permutation of the
    ids plus N(0, 0.5^2) noise."""
    teacher = zipf_teacher(ntok, V, 1.1, 0.5, seed * 1000 + 1, device, shared_perm)
    return dict(teacher=teacher, k=k)


def kl_large(device, seed: int = 4, ntok: int = 8192, V: int = 128256, k: int = 128):
    """Distillation KL: student ~ N(0, 2^2); k distinct uniform teacher ids per
    row with probabilities from N(0, 1.5^2); coef = 1024 / ntok."""
    student = normal_logits(ntok, V, 2.0, seed * 1000 + 1, device)
    ids = distinct_ids(ntok, V, k, seed * 1000 + 2, device)
    probs = softmax_probs(ntok, k, 1.5, seed * 1000 + 3, device)
    return dict(logits=student, ids=ids, probs=probs, coef=1024.0 / ntok)


def kl_bf16_sliced(device, seed: int = 5, ntok: int = 16384, V: int = 151936,
                   k: int = 256, hs: int = 1024):
    """Large-vocabulary bf16 distillation: student and teacher logits are bf16
    casts of independent N(0, 2^2) draws; the teacher's top-k is taken by the
    top-k call; two vocabulary slices' input gradients ``[ntok][hs]`` float32
    ~ N(0, 1) are summed by the slice accumulate.  coef = 1024 / ntok."""
    student = normal_logits(ntok, V, 2.0, seed * 1000 + 1, device, torch.bfloat16)
    teacher = normal_logits(ntok, V, 2.0, seed * 1000 + 2, device, torch.bfloat16)
    g = _gen(seed * 1000 + 3, device)
    dh0 = torch.randn((ntok, hs), generator=g, device=device)
    dh1 = torch.randn((ntok, hs), generator=g, device=device)
    return dict(logits=student, teacher=teacher, k=k, coef=1024.0 / ntok,
                dh0=dh0, dh1=dh1)


# ---------------------------------------------------------------------------
# Inputs of the two tests printed on the pages.

def _page_kl_draws(seed: int):
    """Seeded draws at the shapes of the cortiq-engine ``train_head.rs`` test
    ``head_kl_matches_host`` (V=1024, hs=256, 45 tokens, k=16): head weights
    ~ N(0, 1/hs) [V][hs] and hidden rows ~ N(0, 1) [45][hs] as float32, k
    distinct uniform teacher ids per row, and probabilities
    softmax(N(0, 1)) in float64, cast to float32."""
    V, hs, ntok, k = 1024, 256, 45, 16
    r = np.random.default_rng(seed)
    w = (r.standard_normal((V, hs)) * (1.0 / hs) ** 0.5).astype(np.float32)
    x = r.standard_normal((ntok, hs)).astype(np.float32)
    ids = np.stack([r.permutation(V)[:k] for _ in range(ntok)]).astype(np.int32)
    z = r.standard_normal((ntok, k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    probs = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return w, x, ids, probs


def page_ce_tiny():
    """aprender-train ``wgpu_cross_entropy.rs`` test: 4 tokens, vocabulary 8,
    logits sin(0.3 i) in float32, labels [2, 5, 1, 7], every token in the loss,
    backward scale 1/4."""
    i = np.arange(32, dtype=np.float32)
    logits = np.sin(i * np.float32(0.3)).astype(np.float32).reshape(4, 8)
    labels = np.array([2, 5, 1, 7], dtype=np.int32)
    return dict(logits=logits, labels=labels, rng=(4, 0, 4), scale=0.25)


def page_head_tiny():
    """The shapes of the cortiq-engine ``train_head.rs`` test
    ``head_kl_matches_host``: V=1024, hs=256, 45 tokens, k=16, gscale 256,
    total 45, chunks of 32 rows; the values are this module's own seeded
    draws (``_page_kl_draws``), float32 (each side rounds them to f16
    itself)."""
    w, x, ids, probs = _page_kl_draws(7001)
    return dict(x=x, w=w, ids=ids, probs=probs, total=x.shape[0], gscale=256.0, chunk=32)


def head_inputs(ntok: int, V: int, hs: int, k: int, seed: int, device, wdtype=torch.bfloat16):
    """Vocabulary head inputs: hidden rows x ~ N(0, 1) float32 [ntok][hs];
    head weights ~ N(0, 1/hs) [V][hs] rounded once to ``wdtype`` (the head is
    frozen and stored in half precision); k distinct uniform teacher ids per
    row with probabilities softmax(N(0, 1.5^2)) (float64, cast to float32)."""
    g = _gen(seed, device)
    x = torch.randn((ntok, hs), generator=g, device=device)
    w = (torch.randn((V, hs), generator=g, device=device) * (1.0 / hs) ** 0.5).to(wdtype)
    ids = distinct_ids(ntok, V, k, seed + 1, device)
    probs = softmax_probs(ntok, k, 1.5, seed + 2, device)
    return dict(x=x, w=w, ids=ids, probs=probs)


def page_kl_tiny():
    """The KL rows of the head case above with the logits handed over
    directly: the draws of ``_page_kl_draws`` with the head and hidden rows
    rounded to f16, multiplied in float64 and rounded to float32; coef =
    gscale / total with gscale 256 and total 45."""
    w, x, ids, probs = _page_kl_draws(7001)
    w = w.astype(np.float16).astype(np.float64)
    x = x.astype(np.float16).astype(np.float64)
    logits = (x @ w.T).astype(np.float32)
    return dict(logits=logits, ids=ids, probs=probs, coef=256.0 / x.shape[0])


def to_host_bytes(t: torch.Tensor) -> np.ndarray:
    """Host copy of a logits tensor in the form the oracle reads: float32 as
    float32, bf16 as its raw uint16 bit patterns."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()

