#!/usr/bin/env python3
"""Benchmark of the block-retrieval attention step on one MI355X.

A step is the whole hot path for one attention layer -- score_blocks ->
select_topk -> retrieval_attention, one ``brs_retrieval_step`` call -- on
inputs resident in HBM.  Steps rotate over ``--layers`` independent layer
memories (each with its own K, V, representatives and query), as successive
layers of a model would, so that a step's data has left the 256 MB Infinity
Cache through the other layers' traffic before it is read again.

The default run measures three workloads and prints ONE JSON line (stdout):
  * the headline, 128K-token grouped-query decode (InfLLM-style): top-level
    keys, HBM roofline of the step kernel;
  * ``prefill``: the 80K-token chunked prefill (MemLong-style), matrix-core
    roofline of the prefill kernel;
  * ``decode_1m_b8``: the 1M-token, batch-8 decode (RetrievalAttention
    scale), HBM roofline of its attention kernel;
each with per-step median / p10 / p90, its own bounded CPU-oracle baseline,
and the read-bandwidth references measured in the same run.  Progress goes
to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--layers L]

Timing: W untimed warm-up steps, then K steps timed with GPU events, one
after each step (created without the system-scope fence, so they add no
cache flush).  The K steps are enqueued behind a short GPU spin, so they
run back to back on the GPU whatever the host's launch cost; the host's own
enqueue time per step is reported beside them.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
HEADLINE = "infllm_gqa_decode_128k"
EXTRA = (("prefill", "memlong_chunk_prefill_80k"), ("decode_1m_b8", "retrievalattn_gqa_decode_1m_b8"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """hipEvent_t helpers from the HIP runtime (per-launch and per-step timing)."""

    # hipEventDisableSystemFence: timing-only events, without the system-scope
    # cache writeback/invalidate that would otherwise be charged to the work
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e.value

    def record(self, e, stream):
        assert self.hip.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


KERNEL_SOURCES = {
    "attn_step": ("block_retrieval_sparse_amd/csrc/attn_decode.hip", "block_retrieval_sparse_amd/csrc/brs_internal.h",
                  "block_retrieval_sparse_amd/csrc/brs_wave_topk.h"),
    "attn_split_slot": ("block_retrieval_sparse_amd/csrc/attn_decode.hip",
                        "block_retrieval_sparse_amd/csrc/brs_internal.h"),
    "attn_prefill": ("block_retrieval_sparse_amd/csrc/attn_prefill.hip",
                     "block_retrieval_sparse_amd/csrc/brs_internal.h"),
}


def sources_sha256(paths) -> str:
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the main kernel from the committed counter
    summary for this workload, or None when there is none or the kernel's
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != sources_sha256(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mbytes: int, reps: int) -> dict:
    """A plain device-to-device copy of known size, for scaling the HBM
    byte counters (run under the same counter collection as the kernel)."""
    import torch

    n = mbytes << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n, "copy_bytes_written": n, "launches": reps}


# ---------------------------------------------------------------------------
# algorithmic work of an executed step (from the selection it made)


def attended_tokens(N, B, S, W, rows) -> int:
    """Distinct tokens of one (batch, kv head): sinks, window and the selected
    blocks of all its query heads (each token counted once)."""
    import numpy as np

    T = np.zeros(N, dtype=bool)
    T[:min(S, N)] = True
    T[max(N - W, 0):] = True
    nb = N // B
    for b in np.unique(rows):
        if 0 <= b < nb:
            T[b * B:(b + 1) * B] = True
    return int(T.sum())


def executed_idx(w, step):
    """The selection the step's last run wrote; refuses a layer that never ran."""
    idx = step.idx.cpu().numpy()
    if step.hi > step.lo:
        want = min(w.k, step.hi - step.lo)
        valid = (idx >= 0).sum(axis=2)
        assert (valid == want).all(), "a layer's selection was not written by an executed step"
    return idx


def step_bytes(w, step) -> dict:
    """Algorithmic bytes of one executed step, from its own selection."""
    es = w.elem_bytes
    idx = executed_idx(w, step)
    N = step.mem.length
    kv = 0
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            rows = idx[b, 0] if w.rep_mode == "embed" else idx[b, g * w.group:(g + 1) * w.group]
            kv += attended_tokens(N, w.block, w.sinks, w.window, rows) * w.head_dim * es * 2
    nelig = step.hi - step.lo
    if w.rep_mode == "embed":
        reps = w.batch * nelig * w.rep_dim * 2 + w.batch * w.rep_dim * 2
    else:
        reps = w.batch * w.n_kv_heads * nelig * w.reps_per_block * w.rep_dim * es
    q = w.batch * w.n_q_heads * w.n_q * w.head_dim * es
    out = w.batch * w.n_q_heads * w.n_q * w.head_dim * 4
    return {"reps": reps, "kv": kv, "q": q, "out": out, "total": reps + kv + q + out}


def step_flops(w, step) -> float:
    """Algorithmic flops of the attention of one executed step: 2 d for
    q.k and 2 d for p.v per (query, visible attended token)."""
    import numpy as np

    idx = executed_idx(w, step)
    N = step.mem.length
    total = 0
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            rows = idx[b, 0] if w.rep_mode == "embed" else idx[b, h]
            T = np.zeros(N, dtype=bool)
            T[:min(w.sinks, N)] = True
            T[max(N - w.window, 0):] = True
            for blk in np.unique(rows):
                if 0 <= blk < N // w.block:
                    T[blk * w.block:(blk + 1) * w.block] = True
            cum = np.cumsum(T)
            qpos = N - w.n_q + np.arange(w.n_q)
            total += int(cum[qpos].sum())
    return 4.0 * w.head_dim * total


def weighted(per_layer: list, steps: int):
    """Average of per-layer figures over the steps i = 0 .. steps-1 (layer i mod L)."""
    L = len(per_layer)
    counts = [sum(1 for i in range(steps) if i % L == l) for l in range(L)]
    if isinstance(per_layer[0], dict):
        return {k: sum(c * p[k] for c, p in zip(counts, per_layer)) / steps for k in per_layer[0]}
    return sum(c * p for c, p in zip(counts, per_layer)) / steps


def pct(xs, q):
    ys = sorted(xs)
    if not ys:
        return float("nan")
    pos = (len(ys) - 1) * q
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(ys) - 1)
    return ys[lo] + (ys[hi] - ys[lo]) * (pos - lo)


# ---------------------------------------------------------------------------
# workload set-up


def build_layers(w, n_layers, dev, keep_host_inputs=True):
    import torch

    import block_retrieval_sparse_amd as brs
    from block_retrieval_sparse_amd.pipeline import RetrievalStep
    from synth import inputs as I

    layers = []
    t_build, built_bytes = 0.0, 0
    for i in range(n_layers):
        wl = w.scaled(seed=w.seed + 7919 * i)
        x = I.make_all(wl, dev)
        rep_dtype = torch.bfloat16 if w.rep_mode == "embed" else I.torch_dtype(w)
        mem = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, w.n_tokens, w.block, dtype=I.torch_dtype(w),
                           rep_mode=w.rep_mode, reps_per_block=w.reps_per_block, rep_dim=w.rep_dim,
                           rep_dtype=rep_dtype, row_stride=w.stride, device=dev)
        given = x.get("given_reps", x.get("embeds"))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        mem.append(x["k"], x["v"], given)
        if w.rep_mode == "attnscore":
            # no attention history before the first step: every candidate's
            # representatives come from a zero mass (its first R tokens)
            lo, hi = mem.eligible_range(w.sinks, w.window)
            mem.reps_from_mass(mem.new_mass(), lo, hi)
        torch.cuda.synchronize()
        t_build += time.perf_counter() - t0
        built_bytes += 2 * x["k"].numel() * x["k"].element_size()
        step = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k, w.sinks, w.window)
        qrep = x["rq"].reshape(w.batch, -1).contiguous() if w.rep_mode == "embed" else \
            x["q"][:, :, -1, :].contiguous()
        keep = {"q": x["q"], "qrep": qrep}
        if i == 0 and keep_host_inputs:
            keep.update(host_inputs=x)
        else:
            del x
        layers.append((mem, step, keep))
        log(f"{w.name} layer {i}: built {w.n_tokens} tokens x {w.batch * w.n_kv_heads} kv heads")
    return layers, t_build, built_bytes


def spin_cycles_per_ms(hip, stream) -> float:
    """Cycles of torch's GPU spin per millisecond (measured once)."""
    import torch

    a, b = hip.create(), hip.create()
    torch.cuda.synchronize()
    n = 2_000_000
    hip.record(a, stream)
    torch.cuda._sleep(n)
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(a, b)
    hip.destroy(a)
    hip.destroy(b)
    return n / max(ms, 1e-3)


def timed_steps(one, K, hip, stream, cyc_per_ms, host_us_per_step):
    """K steps with an event after each; enqueued behind a GPU spin long
    enough for the host to queue them all.  Returns per-step ms and the
    total (first to last event)."""
    import torch

    ev = [hip.create() for _ in range(K + 1)]
    spin_ms = min(1.5 * K * max(host_us_per_step, 40.0) * 1e-3 + 0.5, 500.0)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(spin_ms * cyc_per_ms))
    hip.record(ev[0], stream)
    for i in range(K):
        one(i)
        hip.record(ev[i + 1], stream)
    torch.cuda.synchronize()
    per = [hip.elapsed_ms(ev[i], ev[i + 1]) for i in range(K)]
    total = hip.elapsed_ms(ev[0], ev[K])
    for e in ev:
        hip.destroy(e)
    return per, total


def kernel_times(one, K, hip):
    """The main kernel's own duration in each of K steps (events attached to
    its launch by the library), run eagerly; also the host's wall time per step."""
    import torch

    evs = [(hip.create(), hip.create()) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        one(i, evs[i])
    host = (time.perf_counter() - t0) / K
    torch.cuda.synchronize()
    ms = [hip.elapsed_ms(a, b) for (a, b) in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    return ms, host


def read_references(hip, stream, dev, gather_bytes: int, chunk_bytes: int) -> dict:
    """Achievable read bandwidth in this run: a contiguous 4 GiB read, and
    ``gather_bytes`` gathered in chunks of ``chunk_bytes`` at random offsets
    of a 4 GiB buffer (the access pattern of retrieved blocks).  Best of 5
    launches each; the buffer is far larger than the 256 MB Infinity Cache."""
    import torch

    from block_retrieval_sparse_amd import _lib

    n = 4 << 30
    buf = torch.empty(n // 4, dtype=torch.float32, device=dev).normal_()
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    never = 0x5BD1E995
    n_chunks = max(1, gather_bytes // chunk_bytes)
    g = torch.Generator(device="cpu").manual_seed(12345)
    offs = torch.randperm(n // chunk_bytes, generator=g)[:n_chunks].to(torch.int64) * chunk_bytes
    offs = offs.to(dev)

    def best(fn, nbytes):
        ts = []
        for _ in range(6):
            a, b = hip.create(), hip.create()
            torch.cuda.synchronize()
            hip.record(a, stream)
            fn()
            hip.record(b, stream)
            torch.cuda.synchronize()
            ts.append(hip.elapsed_ms(a, b))
            hip.destroy(a)
            hip.destroy(b)
        t = min(ts[1:])
        return nbytes / (t * 1e-3) / 1e9, t

    def contiguous():
        _lib.check(_lib.lib.brs_measure_read(buf.data_ptr(), n, None, 1, never, sink.data_ptr(), stream))

    def gathered():
        _lib.check(_lib.lib.brs_measure_read(buf.data_ptr(), chunk_bytes, offs.data_ptr(), n_chunks, never,
                                             sink.data_ptr(), stream))

    c_gbs, c_ms = best(contiguous, n)
    g_gbs, g_ms = best(gathered, n_chunks * chunk_bytes)
    del buf, offs, sink
    torch.cuda.empty_cache()
    return {"contiguous_GB/s": c_gbs, "contiguous_bytes": n,
            "gather_GB/s": g_gbs, "gather_bytes": n_chunks * chunk_bytes, "gather_chunk_bytes": chunk_bytes,
            "note": "brs_measure_read (one workgroup per chunk, non-temporal 16-byte buffer loads), best of 5 launches after one untimed; HIP events around each launch"}


# ---------------------------------------------------------------------------
# CPU oracle baseline


def cpu_baseline(w, layer0, budget_s: float, cache_bytes: float = 4e9, runs: int = 3) -> dict:
    """The oracle (as it stands) on a bounded sample of layer 0's step: the
    median rate of ``runs`` runs of about ``budget_s / runs`` seconds each.

    Single-head problems (scores, top-k, attention) are timed one after
    another, cycling over the query heads of the first (batch, kv head)
    slices that fit in ``cache_bytes`` once converted to float64 (every slice
    of the 128K and 80K workloads; two of the 1M-token one).  Converting a
    slice and building its representatives are untimed."""
    import numpy as np
    import torch

    import oracle.brs_oracle as O

    x = layer0["host_inputs"]
    f = lambda t: t.to(torch.float64).cpu().numpy()  # noqa: E731
    q = f(x["q"])
    n_pairs = w.batch * w.n_q_heads
    slice_bytes = 2 * w.n_tokens * w.head_dim * 8
    n_slices = max(1, min(w.batch * w.n_kv_heads, int(cache_bytes // slice_bytes)))
    slices = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)][:n_slices]
    cache, cached = {}, 0.0

    def load(b0, g0):
        nonlocal cached
        if (b0, g0) in cache:
            return cache[(b0, g0)]
        K = f(x["k"][b0:b0 + 1, g0:g0 + 1])
        V = f(x["v"][b0:b0 + 1, g0:g0 + 1])
        if w.rep_mode in ("given", "embed"):
            src = x["given_reps"] if w.rep_mode == "given" else x["embeds"]
            reps = f(src[b0:b0 + 1, :1] if w.rep_mode == "embed" else src[b0:b0 + 1, g0:g0 + 1])
        elif w.rep_mode == "attnscore":  # zero mass before the first step, as the GPU side builds them
            nb = K.shape[2] // w.block
            reps = O.reps_attnscore(K[0, 0], np.zeros(K.shape[2]), w.block, w.reps_per_block,
                                    list(range(nb)))[None, None]
        else:
            reps = O.build_reps(K[0, 0], w.rep_mode, w.block, w.reps_per_block, w.dtype)[None, None]
        rq = f(x["rq"]).reshape(w.batch, -1)[b0:b0 + 1] if w.rep_mode == "embed" else None
        item = (K, V, reps, rq)
        size = K.nbytes + V.nbytes + reps.nbytes
        if cached + size <= cache_bytes:
            cache[(b0, g0)] = item
            cached += size
        return item

    pairs = [(b0, g0, h) for (b0, g0) in slices for h in range(g0 * w.group, (g0 + 1) * w.group)]
    rates, done_all, el_all = [], 0, 0.0
    cursor = 0
    for _ in range(runs):
        done, elapsed = 0, 0.0
        while elapsed < budget_s / runs:
            b0, g0, h = pairs[cursor % len(pairs)]
            cursor += 1
            K, V, reps, rq = load(b0, g0)
            t0 = time.perf_counter()
            O.step(q[b0:b0 + 1, h:h + 1], K, V, reps, block=w.block, k=w.k, sinks=w.sinks, window=w.window,
                   mode=w.rep_mode, rq=rq)
            elapsed += time.perf_counter() - t0
            done += 1
        rates.append(w.batch * w.n_q * (done / n_pairs) / elapsed)
        done_all += done
        el_all += elapsed
        log(f"{w.name}: oracle run {len(rates)}: {done} problems in {elapsed:.1f} s")
    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    unit = "query tokens/s" if w.n_q > 1 else "tokens/s"
    what = f"single-head {w.n_q}-query chunk" if w.n_q > 1 else "single-head decode"
    return {"value": sorted(rates)[len(rates) // 2], "unit": unit, "cores": cores, "kind": "oracle",
            "runs": [round(r, 4) for r in rates],
            "sample": f"median of {runs} runs: {done_all} {what} problems (scores, top-k, attention) of layer 0, "
                      f"cycling over the {len(pairs)} query heads of its first {len(slices)} of "
                      f"{w.batch * w.n_kv_heads} (batch, kv head) slices = {done_all / n_pairs:.2f} whole steps of "
                      f"{n_pairs} heads in {el_all:.1f} s of oracle time; float64 conversion and representative "
                      f"builds untimed"}


# ---------------------------------------------------------------------------
# one workload


def run_workload(w, args, hip, stream, cyc_per_ms, headline: bool) -> dict:
    import torch

    from block_retrieval_sparse_amd import _lib

    dev = "cuda:0"
    prefill = w.n_q > 1
    es = w.elem_bytes
    est = (w.batch * w.n_kv_heads * (w.sinks + w.window + w.k * w.group * w.block) * w.head_dim * es * 2)
    n_layers = args.layers or max(1, min(8, math.ceil(1.5e9 / max(est, 1))))
    layers, t_build, built_bytes = build_layers(w, n_layers, dev, keep_host_inputs=not args.no_cpu_baseline)

    def one(i, ev=None):
        mem, step, keep = layers[i % n_layers]
        step.run(keep["q"], keep["qrep"], profile_events=ev)

    t0 = time.perf_counter()
    for i in range(args.warmup):
        one(i)
    host_warm = (time.perf_counter() - t0) / max(args.warmup, 1)
    torch.cuda.synchronize()

    # the timed region: K steps back to back on the GPU
    per, total = timed_steps(one, args.steps, hip, stream, cyc_per_ms, host_warm * 1e6)
    ms_step = total / args.steps
    med = pct(per, 0.5)
    log(f"{w.name}: timed {args.steps} steps, {ms_step * 1e3:.2f} us/step mean, median {med * 1e3:.2f} us "
        f"(p10 {pct(per, 0.1) * 1e3:.2f}, p90 {pct(per, 0.9) * 1e3:.2f})")

    # the same steps eagerly, with the main kernel's own begin/end events
    kern, host_step = kernel_times(one, args.steps, hip)
    kern_avg = sum(kern) / len(kern)

    # algorithmic work of the steps actually run (every layer timed has run)
    assert args.steps >= 1
    used = sorted({i % n_layers for i in range(args.steps)})
    per_layer_bytes = [step_bytes(w, layers[l][1]) if l in used else None for l in range(n_layers)]
    avg = weighted([p if p is not None else {k: 0 for k in per_layer_bytes[used[0]]} for p in per_layer_bytes],
                   args.steps)
    step_time = {"median_us": med * 1e3, "p10_us": pct(per, 0.1) * 1e3, "p90_us": pct(per, 0.9) * 1e3,
                 "mean_us": ms_step * 1e3, "host_enqueue_us": host_step * 1e6,
                 "kernel_median_us": pct(kern, 0.5) * 1e3, "kernel_mean_us": kern_avg * 1e3}
    cfg = {"workload": w.name, "batch": w.batch, "context_tokens": w.n_tokens, "q_heads": w.n_q_heads,
           "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block": w.block, "reps_per_block": w.reps_per_block,
           "rep_mode": w.rep_mode, "top_k": w.k, "window": w.window, "sinks": w.sinks, "queries": w.n_q,
           "layers_rotated": n_layers, "parallelism": "none"}
    res = {"config": cfg, "ms_per_step": med, "step_time": step_time}
    if prefill:
        per_flops = [step_flops(w, layers[l][1]) if l in used else 0.0 for l in range(n_layers)]
        flops = weighted(per_flops, args.steps)
        achieved = flops / (kern_avg * 1e-3) / 1e12
        res.update({
            "metric": "chunked-prefill query tokens/s; MFMA utilisation vs bf16 dense peak",
            "value": w.batch * w.n_q / (med * 1e-3),
            "unit": "query tokens/s",
            "roofline": {"bound": "mfma", "kernel": "attn_prefill", "achieved": achieved,
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                         "traffic": measured_traffic(w.name, "attn_prefill"), "flops_per_launch": flops,
                         "avg_launch_us": kern_avg * 1e3},
            "step_mfma": {"flops": flops, "TFLOP/s": flops / (med * 1e-3) / 1e12,
                          "frac": flops / (med * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS},
        })
    else:
        kname = "attn_step" if layers[0][1].k <= 128 else "attn_split_slot"
        split_bytes = avg["kv"] + avg["q"]
        achieved = split_bytes / (kern_avg * 1e-3) / 1e9
        res.update({
            "metric": "retrieval-attn decode tokens/s @128K ctx; achieved HBM GB/s vs peak",
            "value": w.batch / (med * 1e-3),
            "unit": "tokens/s",
            "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": measured_traffic(w.name, kname), "bytes_per_launch": split_bytes,
                         "avg_launch_us": kern_avg * 1e3},
        })
    res["step_hbm"] = {"algorithmic_bytes": avg["total"], "GB/s": avg["total"] / (med * 1e-3) / 1e9,
                       "frac": avg["total"] / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, "parts": avg}
    res["append_build"] = {"bytes": built_bytes, "s": t_build, "GB/s": built_bytes / max(t_build, 1e-9) / 1e9}

    if headline:
        res.update(extra_passes(w, args, layers, hip))
    if not args.no_cpu_baseline:
        log(f"{w.name}: timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(w, layers[0][2], args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def extra_passes(w, args, layers, hip) -> dict:
    """Attention-score representatives (window mass) and pruning of layer 0."""
    import torch

    from block_retrieval_sparse_amd import _lib
    from block_retrieval_sparse_amd.pipeline import RetrievalStep

    out = {}
    # InfLLM "method": the window mass of one call, and one block's
    # representatives from the mass
    if w.rep_mode != "embed" and w.window > 0:
        n_d = min(args.steps, 50)
        mem0, st0, keep0 = layers[0]
        st_l = RetrievalStep(mem0, w.n_q_heads, w.n_q, w.k, w.sinks, w.window, want_lse=True)
        mass = mem0.new_mass()
        kev = [(hip.create(), hip.create()) for _ in range(n_d)]
        for i in range(n_d):
            st_l.run(keep0["q"], keep0["qrep"])
            _lib.check(_lib.lib.brs_profile_next_attention(kev[i][0], kev[i][1]))  # the mass kernel's own events
            mem0.window_mass(keep0["q"], st_l.lse, w.window, mass)
        torch.cuda.synchronize()
        wm_us = sum(hip.elapsed_ms(a_, b_) for (a_, b_) in kev) / n_d * 1e3
        for a_, b_ in kev:
            hip.destroy(a_)
            hip.destroy(b_)
        W_eff = min(w.window, w.n_tokens)
        wm_bytes = w.batch * w.n_kv_heads * W_eff * (w.head_dim * w.elem_bytes + 8) + \
            w.batch * w.n_q_heads * w.n_q * (w.head_dim * w.elem_bytes + 4)
        out["attnscore_reps"] = {
            "window_mass_us": wm_us, "window_mass_bytes": wm_bytes,
            "window_mass_GB/s": wm_bytes / (wm_us * 1e-6) / 1e9,
            "window_mass_frac": wm_bytes / (wm_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "note": "HIP events attached to the brs_window_mass kernel launch (after an attention call with lse); "
                    "bytes = window K rows + mass read/write + queries + lse"}
        del st_l, mass
    # MemLong dynamic memory update: pruning layer 0's memory into a second
    # memory, with seeded random retrieval counts
    if w.batch * w.n_kv_heads * w.n_tokens * w.stride * w.elem_bytes * 2 <= 8e9:
        mem0 = layers[0][0]
        g_ = torch.Generator(device="cpu").manual_seed(w.seed + 17)
        hits = mem0.new_hits()
        hits[:, : mem0.n_blocks] = torch.randint(0, 8, (w.batch, mem0.n_blocks), generator=g_,
                                                 dtype=torch.int32).to(hits.device)
        dst = mem0.like()
        plan = torch.empty(mem0.blocks_stride, dtype=torch.int32, device=hits.device)
        ts = []
        for _ in range(3):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            mem0.prune_into(hits, dst, plan=plan)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        kept_tokens = dst.length
        pb = 2 * (w.batch * w.n_kv_heads * kept_tokens * w.stride * w.elem_bytes * 2)  # K and V, read + write
        p_us = min(ts) * 1e3
        out["prune"] = {"us": p_us, "kept_tokens": kept_tokens, "of_tokens": mem0.length, "bytes": pb,
                        "GB/s": pb / (p_us * 1e-6) / 1e9, "frac": pb / (p_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                        "note": "events around brs_mem_prune (plan kernel + copy kernel) after a synchronize, "
                                "best of 3; bytes = kept K/V rows read and written"}
        del dst, hits, plan
    return out


def offload_pass(w, args, hip, stream) -> dict:
    """InfLLM-style offload at the workload's shape: K/V in pinned host memory,
    a device cache of blocks sized to what one step may need, decode steps
    whose query drifts (q_t = 0.9 q_(t-1) + 0.44 e_t, so consecutive steps
    share most of their selection).  Reports the blocks and bytes copied over
    the host link per step, the fetch kernel's time and link rate (events
    around its launch after a synchronize), and the whole step's time."""
    import torch

    import block_retrieval_sparse_amd as brs
    from block_retrieval_sparse_amd.pipeline import CachedStep
    from synth import inputs as I

    dev = "cuda:0"
    x = I.make_all(w, dev)
    mem = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, w.n_tokens, w.block, dtype=I.torch_dtype(w),
                       rep_mode=w.rep_mode, reps_per_block=w.reps_per_block, row_stride=w.stride, device=dev,
                       host=True)
    mem.append(x["k"], x["v"])
    torch.cuda.synchronize()
    nbt = -(-w.n_tokens // w.block)
    S = min(w.sinks, w.n_tokens)
    ws = max(w.n_tokens - w.window, S)
    n_pages = -(-S // w.block) + (nbt - ws // w.block if ws < w.n_tokens else 0) + w.group * w.k
    cache = brs.BlockCache(mem, n_pages)
    st = CachedStep(mem, cache, w.n_q_heads, w.k, w.sinks, w.window)
    g = torch.Generator(device=dev).manual_seed(w.seed + 99)
    q = x["q"].float()
    n_t = max(args.steps, 10)
    fetch_ms, step_ms, blocks = [], [], []
    for t in range(n_t):
        if t > 0:
            q = 0.9 * q + math.sqrt(1 - 0.81) * torch.randn(q.shape, generator=g, device=dev)
        qb = q.to(I.torch_dtype(w))
        qrep = qb[:, :, -1, :].contiguous()
        torch.cuda.synchronize()
        before = int(cache.fetched.sum())
        e = [hip.create() for _ in range(4)]
        hip.record(e[0], stream)
        st.score(qrep)
        st.select()
        torch.cuda.synchronize()
        hip.record(e[1], stream)
        st.fetch()
        hip.record(e[2], stream)
        st.attend(qb)
        hip.record(e[3], stream)
        torch.cuda.synchronize()
        fetch_ms.append(hip.elapsed_ms(e[1], e[2]))
        step_ms.append(hip.elapsed_ms(e[0], e[1]) + hip.elapsed_ms(e[1], e[3]))
        for ev in e:
            hip.destroy(ev)
        blocks.append(int(cache.fetched.sum()) - before)
    row_bytes = w.stride * w.elem_bytes
    blk_bytes = 2 * w.block * row_bytes  # K and V of one block
    warm = blocks[1:]
    res = {
        "workload": w.name, "pages_per_kv_head": n_pages, "steps": n_t,
        "cold_step": {"blocks_copied": blocks[0], "bytes": blocks[0] * blk_bytes, "fetch_us": fetch_ms[0] * 1e3,
                      "link_GB/s": blocks[0] * blk_bytes / (fetch_ms[0] * 1e-3) / 1e9},
        "steady": {"blocks_copied_per_step": sum(warm) / len(warm),
                   "bytes_per_step": sum(warm) / len(warm) * blk_bytes,
                   "fetch_us_median": pct(fetch_ms[1:], 0.5) * 1e3,
                   "link_GB/s": (sum(warm) * blk_bytes) / (sum(fetch_ms[1:]) * 1e-3) / 1e9,
                   "step_us_median": pct(step_ms[1:], 0.5) * 1e3},
        "note": "K/V in pinned host memory, a device page cache of the blocks one step may need; query drifts "
                "0.9 per step; step = score + select + fetch + attention (events with a synchronize after the "
                "selection, so the fetch is timed alone)",
    }
    del st, cache, mem, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def run(args):
    import torch

    from block_retrieval_sparse_amd import _lib
    from synth import WORKLOADS

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()
    cyc = spin_cycles_per_ms(hip, stream)
    main = WORKLOADS[args.workload]
    res = run_workload(main, args, hip, stream, cyc, headline=True)
    line = {
        "metric": res.pop("metric"),
        "value": res.pop("value"),
        "unit": res.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if main.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) K/V/q with planted blocks; no dataset or weights)",
        "config": res.pop("config"),
    }
    line.update(res)
    # achievable read bandwidth: contiguous, and gathered in chunks of one
    # retrieved block of one kv head
    chunk = main.block * main.stride * main.elem_bytes
    chunk = max(16, chunk // 16 * 16)
    refs = read_references(hip, stream, "cuda:0", 80 << 20, chunk)
    line["read_reference"] = refs
    if "roofline" in line and line["roofline"]["bound"] == "hbm":
        line["roofline"]["frac_of_gather_read"] = line["roofline"]["achieved"] / refs["gather_GB/s"]
        line["roofline"]["frac_of_contiguous_read"] = line["roofline"]["achieved"] / refs["contiguous_GB/s"]
    if args.workload == HEADLINE and not args.only:
        log("offload pass (host memory + device block cache) ...")
        line["offload"] = offload_pass(main, args, hip, stream)
        for key, name in EXTRA:
            sub = run_workload(WORKLOADS[name], args, hip, stream, cyc, headline=False)
            if sub.get("roofline", {}).get("bound") == "hbm":
                sub["roofline"]["frac_of_contiguous_read"] = sub["roofline"]["achieved"] / refs["contiguous_GB/s"]
            line[key] = sub
    line["spin_cycles_per_ms"] = cyc
    line["lib_version"] = _lib.lib.brs_version()
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="measure only --workload (no prefill / 1M keys)")
    ap.add_argument("--layers", type=int, default=0, help="layer memories to rotate over (0 = enough to exceed the cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=9.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run MB-sized device copies (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the path has no multi-GPU part (each (batch, kv head) is "
              "independent; see the sharding notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.copy_calibration, max(args.steps, 1))), flush=True)
        return
    line = run(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
