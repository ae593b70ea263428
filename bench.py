"""Throughput of the fused vocabulary-softmax loss path on one MI355X.

One step is the whole path over one batch of 4096 token rows at V=32000
(float32), inputs resident in HBM:
  1. teacher top-k + renormalisation (k=64) of Zipf-shaped teacher logits;
  2. distillation KL forward + in-place backward of a student batch against
     that top-k (coef 1024/4096);
  3. cross-entropy forward + in-place backward of an LM batch (8 sequences x
     512 tokens, the first 128 tokens of each outside the loss, +6 at the
     label on 30% of rows, scale 1/3072);
  4. slice accumulate of two [4096][1024] float32 input gradients.
The loss calls overwrite their logits with the gradient, so steps after the
first run on the previous step's gradients; their cost does not depend on
the values.

Prints one JSON line.  `value` is logits rows per second of the whole step
over the timed steps; `roofline` is for the step's dominant kernel (the KL,
which moves the most bytes), from HIP events recorded on the launch stream
around its launches inside the timed steps (the other launches carry no
events there: an event between every launch adds ~17 us a step).  `kernels`
gives every kernel from a second pass of as many steps with events around
every launch.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
                    [--workload step|ce_lm|ce_split|topk_zipf|kl_large|kl_large_unsplit|kl_bf16|
                                kl_sliced|head_kl|head_topk|copy_calib]
    python bench.py --pmc-summary <counter_collection.csv> ...

The other workloads time one configuration each at its full size, for
per-kernel rooflines; the default line is the step above.
`copy_calib` times a plain 1 GiB device-to-device copy, the known-size
kernel that scales the HBM byte counters.

`roofline.traffic` is the dominant kernel's HBM bytes per launch as the
FETCH_SIZE and WRITE_SIZE counters read it (two separate rocprofv3 --pmc
runs of this script), each scaled by bytes / counter of the 1 GiB copy.
The figures live in profiles/hbm_traffic_step_4096x32000_f32.md together
with a SHA-256 of the kernel sources they were taken with; when the sources
differ from that hash, traffic is null.  `--pmc-summary` averages a
rocprofv3 counter CSV per kernel and counter, the numbers that file holds.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_step_4096x32000_f32.md")
KERNEL_SOURCES = ("vl_device.hpp", "vl_launch.hpp", "vl_rows.hip", "vl_topk.hip", "vl_acc.hip")
COPY_CALIB_BYTES = 1 << 30

NTOK, V, K_TOPK, HS = 4096, 32000, 64, 1024
NSEQ, SEQ_LEN, PROMPT = 8, 512, 128


def algorithmic_bytes():
    """Bytes each kernel must move per launch (each input read once, each
    output written once)."""
    row = V * 4
    n_in = NSEQ * (SEQ_LEN - PROMPT)
    return {
        # top-k: read the row; write k ids and k probs
        "topk": NTOK * row + NTOK * K_TOPK * 8,
        # KL, row staged on chip: read + write the row; read ids and probs;
        # write the loss
        "kl": NTOK * 2 * row + NTOK * K_TOPK * 8 + NTOK * 4,
        # CE: rows in the loss read + written, rows outside only written;
        # labels read, loss written
        "ce": n_in * 2 * row + (NTOK - n_in) * row + NTOK * 4 + NTOK * 4,
        # slice accumulate: read dst and src, write dst
        "acc": 3 * NTOK * HS * 4,
    }


def make_inputs(dev):
    import torch
    from gen import inputs as gi
    teacher = gi.topk_zipf(dev, ntok=NTOK, V=V, k=K_TOPK)["teacher"]
    kl_student = gi.normal_logits(NTOK, V, 2.0, 4001, dev)
    ce = gi.ce_lm(dev, nseq=NSEQ, seq_len=SEQ_LEN, V=V, prompt=PROMPT)
    g = torch.Generator(device=dev)
    g.manual_seed(4002)
    dh0 = torch.randn((NTOK, HS), generator=g, device=dev)
    dh1 = torch.randn((NTOK, HS), generator=g, device=dev)
    return dict(teacher=teacher, kl_student=kl_student, ce_logits=ce["logits"],
                labels=ce["labels"], rng=ce["rng"], scale=ce["scale"], dh0=dh0, dh1=dh1)


def host_copies(x):
    """Host bytes of the step's inputs, taken before the in-place calls."""
    from gen.inputs import to_host_bytes
    return {k: to_host_bytes(x[k]) for k in ("teacher", "kl_student", "ce_logits", "labels",
                                              "dh0", "dh1")}


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (or the platform's)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_pass(h, rng, scale, rows):
    """Every stage of the step on the first `rows` rows, wall-clock seconds."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    ids, probs = oracle.topk(h["teacher"][:rows], K_TOPK)
    oracle.kl(h["kl_student"][:rows], ids, probs.astype(np.float32), coef=1024.0 / NTOK)
    oracle.ce(h["ce_logits"][:rows], h["labels"][:rows], rng=rng, scale=scale)
    oracle.acc(h["dh0"][:rows], h["dh1"][:rows])
    return time.perf_counter() - t0


def cpu_baseline(h, rng, scale, rows: int, rows_1core: int):
    """The float64 oracle on the host over the first `rows` rows of the same
    inputs, every stage of the step, wall-clock: once on every thread the
    OpenMP runtime uses, once on one thread (the first `rows_1core` rows)."""
    import oracle

    oracle.topk(h["teacher"][:2], K_TOPK)  # load the library outside the timing
    threads = oracle.threads()
    dt = _oracle_pass(h, rng, scale, rows)
    oracle.set_threads(1)
    try:
        dt1 = _oracle_pass(h, rng, scale, rows_1core)
    finally:
        oracle.set_threads(threads)
    return {"value": rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of the {NTOK} rows of every stage (top-k, KL, CE, "
                      f"slice accumulate) at V={V}, float64, {dt:.2f} s wall-clock on "
                      f"{threads} threads",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_core": {"value": rows_1core / dt1, "unit": "rows/s", "cores": 1,
                            "sample": f"first {rows_1core} rows of every stage, "
                                      f"{dt1:.2f} s wall-clock on 1 thread"}}


def workload_cpu_baseline(run, ntok, rows, rows_1core, what):
    """The float64 oracle over the first rows of one configuration, timed on
    every thread the OpenMP runtime uses and on one thread.  `run(n)` runs
    the oracle's stages of the configuration on the first n rows (inputs
    copied to the host before the GPU calls overwrite them)."""
    import oracle
    run(2)  # load the library outside the timing
    threads = oracle.threads()
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        run(rows_1core)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    return {"value": rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of the {ntok} rows ({what}), float64, {dt:.2f} s "
                      f"wall-clock on {threads} threads",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_core": {"value": rows_1core / dt1, "unit": "rows/s", "cores": 1,
                            "sample": f"first {rows_1core} rows, {dt1:.2f} s wall-clock on "
                                      f"1 thread"}}


def other_workload(name, dev):
    """(calls, bytes per call, ntok, config, cpu) of one full-size
    configuration.  Each call is (kernel name, function); cpu is None or a
    function of no arguments that times the oracle on a sample of the same
    inputs (host copies taken here, before any call)."""
    import numpy as np
    import torch
    import vocab_softmax_loss_amd as vl
    from gen import inputs as gi
    from gen.inputs import to_host_bytes

    cpu = None

    if name == "ce_lm":
        c = gi.ce_lm(dev)
        ntok, V = c["logits"].shape
        loss = torch.empty(ntok, device=dev)
        n_in = 8 * 384
        calls = [("ce", lambda: vl.vl_ce_fwd_bwd(c["logits"], c["labels"], loss, rng=c["rng"],
                                                 scale=c["scale"]))]
        nbytes = {"ce": n_in * 2 * V * 4 + (ntok - n_in) * V * 4 + ntok * 8}
        cfg = {"workload": gi.CE_LM.name, "ntok": ntok, "V": V, "dtype": "f32"}
        hx, hl = to_host_bytes(c["logits"]), to_host_bytes(c["labels"])

        def cpu():
            import oracle
            return workload_cpu_baseline(
                lambda n: oracle.ce(hx[:n], hl[:n], rng=c["rng"], scale=c["scale"]),
                ntok, ntok, ntok, "CE loss and gradient")
    elif name == "ce_split":
        # the same configuration through the two-pass calls: forward only,
        # backward from the saved lse, then the mean loss on the device
        c = gi.ce_lm(dev)
        x, lab, rng = c["logits"], c["labels"], c["rng"]
        ntok, V = x.shape
        loss = torch.empty(ntok, device=dev)
        lse = torch.empty(ntok, device=dev)
        mean = torch.empty(1, device=dev)
        n_in = 8 * 384
        calls = [("ce_fwd", lambda: vl.vl_ce_fwd(x, lab, loss, lse, rng=rng)),
                 ("ce_bwd", lambda: vl.vl_ce_bwd(x, lab, lse, rng=rng, scale=c["scale"])),
                 ("mean", lambda: vl.vl_loss_mean(loss, mean, rng=rng))]
        nbytes = {"ce_fwd": n_in * V * 4 + n_in * 4 + ntok * 8,
                  "ce_bwd": n_in * 2 * V * 4 + (ntok - n_in) * V * 4 + n_in * 8,
                  "mean": ntok * 4 + 4}
        cfg = {"workload": gi.CE_LM.name + ", two-pass calls", "ntok": ntok, "V": V,
               "dtype": "f32", "bytes_model": "forward 1R, backward 1R+1W"}
    elif name == "topk_zipf":
        c = gi.topk_zipf(dev)
        t, k = c["teacher"], c["k"]
        ntok, V = t.shape
        ids = torch.empty((ntok, k), dtype=torch.int32, device=dev)
        probs = torch.empty((ntok, k), device=dev)
        calls = [("topk", lambda: vl.vl_topk_renorm(t, k, ids, probs))]
        nbytes = {"topk": ntok * V * 4 + ntok * k * 8}
        cfg = {"workload": gi.TOPK_ZIPF.name, "ntok": ntok, "V": V, "k": k, "dtype": "f32"}
        ht = to_host_bytes(t)

        def cpu():
            import oracle
            return workload_cpu_baseline(lambda n: oracle.topk(ht[:n], k), ntok, ntok, 512,
                                         "top-k and renormalised probabilities")
    elif name in ("kl_large", "kl_large_unsplit"):
        c = gi.kl_large(dev)
        x = c["logits"]
        ntok, V = x.shape
        k = c["ids"].shape[1]
        loss = torch.empty(ntok, device=dev)
        if name == "kl_large":
            # the workspace call: each 128256-value row split over four
            # co-resident workgroups, read once and written once
            ws = torch.empty(vl.vl_split_workspace_bytes(), dtype=torch.uint8, device=dev)
            calls = [("kl", lambda: vl.vl_kl_fwd_bwd_ws(x, c["ids"], c["probs"], loss, ws,
                                                        coef=c["coef"]))]
            model = "1R+1W (rows split over 4 workgroups)"
        else:
            # one workgroup per row: the row does not fit one CU, so the
            # kernel reads about a quarter of it a second time (the rest of
            # pass 2 comes from registers and LDS)
            calls = [("kl", lambda: vl.vl_kl_fwd_bwd(x, c["ids"], c["probs"], loss,
                                                     coef=c["coef"]))]
            model = "1R+1W algorithmic (the kernel re-reads ~27% of each row)"
        nbytes = {"kl": ntok * 2 * V * 4 + ntok * k * 8 + ntok * 4}
        cfg = {"workload": gi.KL_LARGE.name, "ntok": ntok, "V": V, "k": k, "dtype": "f32",
               "bytes_model": model}
        hx = to_host_bytes(x[:4096])
        hi, hp = to_host_bytes(c["ids"][:4096]), to_host_bytes(c["probs"][:4096])

        def cpu():
            import oracle
            return workload_cpu_baseline(
                lambda n: oracle.kl(hx[:n], hi[:n], hp[:n], coef=c["coef"]), ntok, 4096, 512,
                "KL loss and gradient")
    elif name == "kl_bf16":
        c = gi.kl_bf16_sliced(dev)
        x, t, k = c["logits"], c["teacher"], c["k"]
        ntok, V = x.shape
        hs = c["dh0"].shape[1]
        ids = torch.empty((ntok, k), dtype=torch.int32, device=dev)
        probs = torch.empty((ntok, k), device=dev)
        loss = torch.empty(ntok, device=dev)
        calls = [("topk", lambda: vl.vl_topk_renorm(t, k, ids, probs)),
                 ("kl", lambda: vl.vl_kl_fwd_bwd(x, ids, probs, loss, coef=c["coef"])),
                 ("acc", lambda: vl.vl_slice_acc(c["dh0"], c["dh1"]))]
        # the KL holds each 151936-entry bf16 row in registers: read once,
        # written once
        nbytes = {"topk": ntok * V * 2 + ntok * k * 8,
                  "kl": ntok * 2 * V * 2 + ntok * k * 8 + ntok * 4,
                  "acc": 3 * ntok * hs * 4}
        cfg = {"workload": gi.KL_BF16.name, "ntok": ntok, "V": V, "k": k, "dtype": "bf16",
               "bytes_model": "KL 1R+1W"}
        hx, ht = to_host_bytes(x[:1024]), to_host_bytes(t[:1024])
        h0, h1 = to_host_bytes(c["dh0"][:1024]), to_host_bytes(c["dh1"][:1024])

        def cpu():
            import oracle

            def run(n):
                oi, op = oracle.topk(ht[:n], k)
                oracle.kl(hx[:n], oi, op.astype(np.float32), coef=c["coef"])
                oracle.acc(h0[:n], h1[:n])
            return workload_cpu_baseline(run, ntok, 1024, 64,
                                         "teacher top-k, KL loss and gradient, slice "
                                         "accumulate of the row's 1024 values")
    elif name == "kl_sliced":
        # the same bf16 workload as two vocabulary slices of 75968, each its
        # own [ntok][75968] buffer: statistics of each slice, the merge, the
        # gradient of each slice from the merged lse, then the slice
        # accumulate of the two slices' input gradients
        c = gi.kl_bf16_sliced(dev)
        x, t, k = c["logits"], c["teacher"], c["k"]
        ntok, V = x.shape
        hs = c["dh0"].shape[1]
        ids = torch.empty((ntok, k), dtype=torch.int32, device=dev)
        probs = torch.empty((ntok, k), device=dev)
        vl.vl_topk_renorm(t, k, ids, probs)
        del t, c["teacher"]
        w = V // 2
        sl = [x[:, :w].contiguous(), x[:, w:].contiguous()]
        del x, c["logits"]
        parts = torch.empty((2, ntok, 4), device=dev)
        loss = torch.empty(ntok, device=dev)
        lse = torch.empty(ntok, device=dev)
        calls = [("part0", lambda: vl.vl_kl_slice_fwd(sl[0], 0, ids, probs, parts[0])),
                 ("part1", lambda: vl.vl_kl_slice_fwd(sl[1], w, ids, probs, parts[1])),
                 ("merge", lambda: vl.vl_kl_slice_merge(parts, loss, lse)),
                 ("bwd0", lambda: vl.vl_kl_slice_bwd(sl[0], 0, ids, probs, lse,
                                                     coef=c["coef"])),
                 ("bwd1", lambda: vl.vl_kl_slice_bwd(sl[1], w, ids, probs, lse,
                                                     coef=c["coef"])),
                 ("acc", lambda: vl.vl_slice_acc(c["dh0"], c["dh1"]))]
        # the part pass reads its slice once; the gradient pass reads and
        # writes it; ids and probs are read by each pass of each slice
        nbytes = {"part0": ntok * w * 2 + ntok * k * 8 + ntok * 16,
                  "part1": ntok * w * 2 + ntok * k * 8 + ntok * 16,
                  "merge": 2 * ntok * 16 + ntok * 8,
                  "bwd0": ntok * 2 * w * 2 + ntok * k * 8 + ntok * 4,
                  "bwd1": ntok * 2 * w * 2 + ntok * k * 8 + ntok * 4,
                  "acc": 3 * ntok * hs * 4}
        cfg = {"workload": gi.KL_BF16.name + ", two vocabulary slices of 75968 in separate "
                           "buffers", "ntok": ntok, "V": V, "k": k, "dtype": "bf16",
               "bytes_model": "slice statistics 1R, slice gradient 1R+1W"}
    elif name == "head_kl":
        # the vocabulary head around the KL: two GEMMs of 2 ntok V hs flops
        # each on the matrix cores, the KL rows and two conversions between.
        # The whole batch is one chunk (15 GB of scratch): larger products
        # run faster (chunks of 4096 rows: 13.7-14.0 ms a call; 8192: 12.8;
        # 16384: 12.7).
        c = gi.head_inputs(16384, 151936, 1024, 256, 6001, dev, torch.bfloat16)
        ntok, hs = c["x"].shape
        V, k, chunk, gscale = c["w"].shape[0], c["ids"].shape[1], ntok, 1024.0
        dx = torch.empty((ntok, hs), device=dev)
        loss = torch.empty(ntok, device=dev)
        scratch = torch.empty(vl.vl_head_scratch_bytes(chunk, V, hs), dtype=torch.uint8,
                              device=dev)
        # set-up, before the warm-up: pick the dx product's hipBLASLt
        # algorithm for this shape (the call waits while it times them)
        vl.vl_head_kl(c["x"], c["w"], c["ids"], c["probs"], dx, loss, ntok, gscale, chunk,
                      scratch, tune=True)
        calls = [("head", lambda: vl.vl_head_kl(c["x"], c["w"], c["ids"], c["probs"], dx, loss,
                                                ntok, gscale, chunk, scratch))]
        nbytes = {"head": None}
        cfg = {"workload": "head_16384x151936x1024_bf16_k256", "ntok": ntok, "V": V, "hs": hs,
               "k": k, "chunk": chunk, "dtype": "bf16", "flops": 2 * 2 * ntok * V * hs}
    elif name == "head_topk":
        # the teacher side of the head: the logits product on the matrix
        # cores, then the top-k rows over the float32 logits, one chunk
        c = gi.head_inputs(16384, 151936, 1024, 4, 6002, dev, torch.bfloat16)
        ntok, hs = c["x"].shape
        V, k, chunk = c["w"].shape[0], 256, ntok
        ids = torch.empty((ntok, k), dtype=torch.int32, device=dev)
        probs = torch.empty((ntok, k), device=dev)
        scratch = torch.empty(vl.vl_head_topk_scratch_bytes(chunk, V, hs), dtype=torch.uint8,
                              device=dev)
        vl.vl_head_topk(c["x"], c["w"], k, ids, probs, chunk, scratch, tune=True)
        calls = [("head_topk", lambda: vl.vl_head_topk(c["x"], c["w"], k, ids, probs, chunk,
                                                       scratch))]
        nbytes = {"head_topk": None}
        cfg = {"workload": "head_topk_16384x151936x1024_bf16_k256", "ntok": ntok, "V": V,
               "hs": hs, "k": k, "chunk": chunk, "dtype": "bf16", "flops": 2 * ntok * V * hs}
    elif name == "copy_calib":
        n = COPY_CALIB_BYTES // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        calls = [("copy", lambda: dst.copy_(src))]
        nbytes = {"copy": 2 * COPY_CALIB_BYTES}
        ntok = 1
        cfg = {"workload": "plain device copy of 1 GiB float32 (counter calibration)",
               "bytes": COPY_CALIB_BYTES, "dtype": "f32"}
    else:
        raise SystemExit(f"unknown workload {name}")
    return calls, nbytes, ntok, cfg, cpu


def kernel_sources_sha256():
    """SHA-256 over the HIP kernel sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "vocab_softmax_loss_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` in the step, from the counter file,
    or None when the file is missing, lacks the kernel or was taken with
    other kernel sources."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"^kernel_sources_sha256: ([0-9a-f]{64})$", text, re.M)
    if not m or m.group(1) != kernel_sources_sha256():
        return None
    m = re.search(rf"^traffic_bytes\.{kernel}: (\d+)$", text, re.M)
    return int(m.group(1)) if m else None


def pmc_summary(paths):
    """Per kernel and counter: dispatches and mean value, from rocprofv3
    counter_collection CSVs."""
    import csv
    from collections import defaultdict
    acc = defaultdict(list)
    for p in paths:
        with open(p) as fh:
            for r in csv.DictReader(fh):
                acc[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    for (kern, ctr), v in sorted(acc.items()):
        print(f"{ctr}\t{len(v)}\t{sum(v) / len(v):.1f}\t{kern}")


def time_calls(calls, steps, warmup):
    """Average ms per call (HIP events on the current stream around every
    launch) and per sequence of all calls."""
    import torch
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    n = len(calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        for i, (_, fn) in enumerate(calls):
            ev[s][i].record()
            fn()
        ev[s][n].record()
    t1.record()
    torch.cuda.synchronize()
    per = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
           for i, (name, _) in enumerate(calls)}
    return per, t0.elapsed_time(t1) / steps


def time_step(calls, steps, warmup, dom):
    """The timed region of the step: `steps` steps between two
    synchronisations, with HIP events only around the launches of the
    dominant kernel `dom` (events between every launch add ~17 us a step of
    their own).  Returns (ms per step, `dom`'s average ms per launch)."""
    import torch
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        for name, fn in calls:
            if name == dom:
                ev[s][0].record()
                fn()
                ev[s][1].record()
            else:
                fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, sum(a.elapsed_time(b) for a, b in ev) / steps


MFMA_PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/f16 matrix peak


def kernel_table(per_ms, nbytes, ntok):
    out = {}
    for n, ms in per_ms.items():
        if nbytes[n] is None:
            out[n] = {"ms": round(ms, 5), "rows/s": round(ntok / (ms * 1e-3), 1)}
            continue
        gbs = nbytes[n] / (ms * 1e-3) / 1e9
        out[n] = {"ms": round(ms, 5), "bytes": nbytes[n], "GB/s": round(gbs, 1),
                  "frac": round(gbs / HBM_PEAK_GBS, 4), "rows/s": round(ntok / (ms * 1e-3), 1)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=NTOK)
    ap.add_argument("--cpu-rows-1core", type=int, default=512)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default="step")
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs on a single MI355X "
              "(token rows shard across GPUs with no exchange between them).", file=sys.stderr)
        sys.exit(2)

    import torch
    import vocab_softmax_loss_amd as vl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.workload != "step":
        calls, nbytes, ntok, cfg, cpu = other_workload(args.workload, dev)
        per, seq_ms = time_calls(calls, args.steps, args.warmup)
        kernels = kernel_table(per, nbytes, ntok)
        dom = max(per, key=per.get)
        if "flops" in cfg:
            # matrix-core bound: the whole call's flops over its time
            tf = cfg["flops"] / (per[dom] * 1e-3) / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(tf, 1),
                    "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_PEAK_BF16_TFLOPS, 4), "traffic": None}
        else:
            roof = {"kernel": dom, "bound": "hbm", "achieved": kernels[dom]["GB/s"],
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom]["frac"],
                    "traffic": None}
        print(json.dumps({
            "metric": f"rows/s and achieved HBM GB/s of one configuration ({args.workload})",
            "value": round(ntok / (seq_ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(seq_ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": cfg["dtype"], "data": "synthetic", "config": cfg,
            "roofline": roof, "kernels": kernels,
            "cpu_baseline": None if (cpu is None or args.no_cpu) else cpu()}), flush=True)
        return
    x = make_inputs(dev)
    host = None if args.no_cpu else host_copies(x)
    ids = torch.empty((NTOK, K_TOPK), dtype=torch.int32, device=dev)
    probs = torch.empty((NTOK, K_TOPK), device=dev)
    kl_loss = torch.empty(NTOK, device=dev)
    ce_loss = torch.empty(NTOK, device=dev)
    coef = 1024.0 / NTOK
    calls = [
        ("topk", lambda: vl.vl_topk_renorm(x["teacher"], K_TOPK, ids, probs)),
        ("kl", lambda: vl.vl_kl_fwd_bwd(x["kl_student"], ids, probs, kl_loss, coef=coef)),
        ("ce", lambda: vl.vl_ce_fwd_bwd(x["ce_logits"], x["labels"], ce_loss, rng=x["rng"],
                                        scale=x["scale"])),
        ("acc", lambda: vl.vl_slice_acc(x["dh0"], x["dh1"])),
    ]
    # The dominant kernel: the one that moves the most bytes (the KL).
    alg = algorithmic_bytes()
    dom = max(alg, key=alg.get)
    ms_per_step, dom_ms = time_step(calls, args.steps, args.warmup, dom)
    dom_gbs = alg[dom] / (dom_ms * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom)}
    # Every kernel, from a second pass of as many steps with events around
    # every launch.
    per_kernel_ms, _ = time_calls(calls, args.steps, 0)
    kernels = kernel_table(per_kernel_ms, alg, NTOK)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(host, x["rng"], x["scale"], min(args.cpu_rows, NTOK),
                           min(args.cpu_rows_1core, NTOK))

    out = {
        "metric": "logits rows/s + achieved HBM GB/s (% of peak), fused CE/KL fwd+bwd at "
                  "V=32000",
        "value": round(NTOK / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "teacher top-k (k=64) + distillation KL fwd+bwd + CE fwd+bwd "
                               "(8x512 tokens, prompt 128 masked) + slice accumulate, "
                               "4096 rows x V=32000 float32",
                   "ntok": NTOK, "V": V, "k": K_TOPK, "seq_len": SEQ_LEN,
                   "loss_range": [PROMPT, SEQ_LEN], "slice_acc": [NTOK, HS]},
        "roofline": roofline,
        "kernels": kernels,
        "kernels_pass": "a second pass of the same steps, HIP events around every launch",
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
