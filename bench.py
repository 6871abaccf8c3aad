#!/usr/bin/env python3
"""Benchmark of one block-retrieval attention step on one MI355X.

A step is the whole hot path for one attention layer: score_blocks ->
select_topk -> retrieval_attention, on inputs resident in HBM.  Steps rotate
over ``--layers`` independent layer memories (each with its own K, V,
representatives and query), as successive layers of a model would, so that a
step's data has been evicted from the 256 MB Infinity Cache by the other
layers' traffic before it is read again.

Prints one JSON line (stdout).  Progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--layers L]
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs from the HIP runtime (for per-launch kernel timing)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    # hipEventDisableSystemFence: timing-only events, without the system-scope
    # cache writeback/invalidate that would otherwise be charged to the kernel
    DISABLE_SYSTEM_FENCE = 0x20000000

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e.value

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
    "attn_prefill": ("block_retrieval_sparse_amd/csrc/attn_prefill.hip",
                     "block_retrieval_sparse_amd/csrc/brs_internal.h"),
}


def sources_sha256(paths=KERNEL_SOURCES["attn_step"]) -> str:
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str = "attn_step"):
    """HBM bytes per launch of the main attention kernel from the committed
    counter summary for this workload, or None when there is none or the
    kernel's sources have changed since the counters were taken."""
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


def build_layers(w, n_layers, dev):
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
        if i == 0:
            keep.update(host_inputs=x)
        else:
            del x
        layers.append((mem, step, keep))
        log(f"layer {i}: built {w.n_tokens} tokens x {w.batch * w.n_kv_heads} kv heads")
    return layers, t_build, built_bytes


def step_bytes(w, step) -> dict:
    """Algorithmic bytes of one executed step, from its own selection."""
    es = 4 if w.dtype == "f32" else 2
    idx = step.idx.cpu().numpy()
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

    idx = step.idx.cpu().numpy()
    N = step.mem.length
    pos = np.arange(N)
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


def cpu_baseline(w, layer0, budget_s: float, cache_bytes: float = 4e9) -> dict:
    """The oracle (as it stands) on a bounded sample of layer 0's step.

    Decode problems (one query head each: scores, top-k, attention) are timed
    one after another, cycling over the (batch, query head) pairs, until about
    ``budget_s`` seconds of oracle work are done.  Converting a (batch, kv
    head) slice to float64 and building its representatives are untimed; up
    to ``cache_bytes`` of converted slices are kept for later cycles."""
    import numpy as np
    import torch

    import oracle.brs_oracle as O

    x = layer0["host_inputs"]
    f = lambda t: t.to(torch.float64).cpu().numpy()  # noqa: E731
    q = f(x["q"])
    n_pairs = w.batch * w.n_q_heads
    slices = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
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

    done, elapsed = 0, 0.0
    while elapsed < budget_s:
        for (b0, g0) in slices:
            K, V, reps, rq = load(b0, g0)
            for h in range(g0 * w.group, (g0 + 1) * w.group):
                t0 = time.perf_counter()
                O.step(q[b0:b0 + 1, h:h + 1], K, V, reps, block=w.block, k=w.k, sinks=w.sinks, window=w.window,
                       mode=w.rep_mode, rq=rq)
                elapsed += time.perf_counter() - t0
                done += 1
                if elapsed >= budget_s:
                    break
            if elapsed >= budget_s:
                break
    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    steps = done / n_pairs
    unit = "query tokens/s" if w.n_q > 1 else "tokens/s"
    what = f"single-head {w.n_q}-query chunk" if w.n_q > 1 else "single-head decode"
    return {"value": w.batch * w.n_q * steps / elapsed, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{done} {what} problems (scores, top-k, attention) of layer 0, cycling over "
                      f"its {n_pairs} (batch, query head) pairs = {steps:.2f} whole steps in {elapsed:.1f} s of "
                      f"oracle time; float64 conversion and representative builds untimed"}


def run(args):
    import torch

    from block_retrieval_sparse_amd import _lib
    from synth import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    prefill = w.n_q > 1
    es = 4 if w.dtype == "f32" else 2
    est = (w.batch * w.n_kv_heads * (w.sinks + w.window + w.k * w.group * w.block) * w.head_dim * es * 2)
    n_layers = args.layers or max(1, min(8, math.ceil(1.5e9 / max(est, 1))))
    layers, t_build, built_bytes = build_layers(w, n_layers, dev)

    def one(i, ev=None):
        mem, step, keep = layers[i % n_layers]
        step.run(keep["q"], keep["qrep"], profile_events=ev)

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    per_layer = [step_bytes(w, st) for (_, st, _) in layers]
    avg = {k: sum(p[k] for p in per_layer) / n_layers for k in per_layer[0]}

    # pass A: the timed region
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s0.record()
    for i in range(args.steps):
        one(i)
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = s0.elapsed_time(s1)
    ms_step = ms_total / args.steps
    log(f"timed {args.steps} steps: {ms_step * 1e3:.2f} us/step (host wall {wall * 1e3 / args.steps:.2f} us/step)")

    # pass B: the same steps with the attention kernel's own begin/end timestamps
    he = HipEvents()
    evs = [(he.create(), he.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        one(i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [he.elapsed_ms(a, b) for (a, b) in evs]
    for a, b in evs:
        he.destroy(a)
        he.destroy(b)
    kern_avg = sum(kern_ms) / len(kern_ms)

    # pass C: per-stage breakdown (events on the library's stream = torch's current stream)
    stage = {"score": 0.0, "select": 0.0, "attend": 0.0}
    n_c = min(args.steps, 100)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4 * n_c)]
    for i in range(n_c):
        mem, step, keep = layers[i % n_layers]
        ev[4 * i].record()
        step.score(keep["qrep"])
        ev[4 * i + 1].record()
        step.select()
        ev[4 * i + 2].record()
        step.attend(keep["q"])
        ev[4 * i + 3].record()
    torch.cuda.synchronize()
    for i in range(n_c):
        stage["score"] += ev[4 * i].elapsed_time(ev[4 * i + 1]) / n_c
        stage["select"] += ev[4 * i + 1].elapsed_time(ev[4 * i + 2]) / n_c
        stage["attend"] += ev[4 * i + 2].elapsed_time(ev[4 * i + 3]) / n_c

    # pass D: attention-score representatives (InfLLM "method"): the window
    # mass of one call, and one block's representatives from the mass
    mass_res = None
    if w.rep_mode != "embed" and w.window > 0:
        from block_retrieval_sparse_amd.pipeline import RetrievalStep

        n_d = min(args.steps, 50)
        mem0, st0, keep0 = layers[0]
        st_l = RetrievalStep(mem0, w.n_q_heads, w.n_q, w.k, w.sinks, w.window, want_lse=True)
        mass = mem0.new_mass()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_d)]
        kev = [(he.create(), he.create()) for _ in range(n_d)]
        b_last = mem0.n_blocks - 1
        for i in range(n_d):
            st_l.run(keep0["q"], keep0["qrep"])
            _lib.check(_lib.lib.brs_profile_next_attention(kev[i][0], kev[i][1]))  # the mass kernel's own events
            mem0.window_mass(keep0["q"], st_l.lse, w.window, mass)
            if w.rep_mode == "attnscore":
                torch.cuda.synchronize()
                ev[2 * i].record()
                mem0.reps_from_mass(mass, b_last, b_last + 1)
                ev[2 * i + 1].record()
        torch.cuda.synchronize()
        wm_us = sum(he.elapsed_ms(a_, b_) for (a_, b_) in kev) / n_d * 1e3
        for a_, b_ in kev:
            he.destroy(a_)
            he.destroy(b_)
        W_eff = min(w.window, w.n_tokens)
        es_ = 4 if w.dtype == "f32" else 2
        wm_bytes = w.batch * w.n_kv_heads * W_eff * (w.head_dim * es_ + 8) + \
            w.batch * w.n_q_heads * w.n_q * (w.head_dim * es_ + 4)
        mass_res = {"window_mass_us": wm_us, "window_mass_bytes": wm_bytes,
                    "window_mass_GB/s": wm_bytes / (wm_us * 1e-6) / 1e9,
                    "window_mass_frac": wm_bytes / (wm_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "note": "HIP events attached to the brs_window_mass kernel launch (after an attention call "
                            "with lse); bytes = window K rows + mass read/write + queries + lse"}
        if w.rep_mode == "attnscore":
            mass_res["reps_from_mass_us"] = sum(ev[2 * i].elapsed_time(ev[2 * i + 1])
                                                for i in range(n_d)) / n_d * 1e3
            mass_res["reps_from_mass_note"] = "one block per call, events around the call after a synchronize"
        del st_l, mass

    # pass E: pruning on overflow (MemLong dynamic memory update) of layer 0's
    # memory into a second memory, with seeded random retrieval counts
    prune_res = None
    if w.batch * w.n_kv_heads * w.n_tokens * w.stride * (4 if w.dtype == "f32" else 2) * 2 <= 8e9:
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
        es_ = 4 if w.dtype == "f32" else 2
        kept_tokens = dst.length
        pb = 2 * (w.batch * w.n_kv_heads * kept_tokens * w.stride * es_ * 2)  # K and V, read + write
        p_us = min(ts) * 1e3
        prune_res = {"us": p_us, "kept_tokens": kept_tokens, "of_tokens": mem0.length, "bytes": pb,
                     "GB/s": pb / (p_us * 1e-6) / 1e9, "frac": pb / (p_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "note": "events around brs_mem_prune (plan kernel + copy kernel) after a synchronize, best of 3; "
                             "bytes = kept K/V rows read and written"}
        del dst, hits, plan

    split_bytes = avg["kv"] + avg["q"]
    cfg = {"workload": w.name, "batch": w.batch, "context_tokens": w.n_tokens, "q_heads": w.n_q_heads,
           "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block": w.block, "reps_per_block": w.reps_per_block,
           "rep_mode": w.rep_mode, "top_k": w.k, "window": w.window, "sinks": w.sinks, "queries": w.n_q,
           "layers_rotated": n_layers, "parallelism": "none"}
    res = {
        "metric": "retrieval-attn decode tokens/s @128K ctx; achieved HBM GB/s vs peak",
        "value": w.batch / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) K/V/q with planted blocks; no dataset or weights)",
        "config": cfg,
    }
    if prefill:
        flops = sum(step_flops(w, st) for (_, st, _) in layers) / n_layers
        achieved = flops / (kern_avg * 1e-3) / 1e12
        res.update({
            "metric": "chunked-prefill query tokens/s; MFMA utilisation vs bf16 dense peak",
            "value": w.batch * w.n_q / (ms_step * 1e-3),
            "unit": "query tokens/s",
            "roofline": {"bound": "mfma", "kernel": "attn_prefill", "achieved": achieved,
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                         "traffic": measured_traffic(w.name, "attn_prefill"), "flops_per_launch": flops,
                         "avg_launch_us": kern_avg * 1e3},
            "step_mfma": {"flops": flops, "TFLOP/s": flops / (ms_step * 1e-3) / 1e12,
                          "frac": flops / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS},
        })
    else:
        achieved = split_bytes / (kern_avg * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": "attn_step", "achieved": achieved, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(w.name),
                           "bytes_per_launch": split_bytes, "avg_launch_us": kern_avg * 1e3}
    res.update({
        "step_hbm": {"algorithmic_bytes": avg["total"], "GB/s": avg["total"] / (ms_step * 1e-3) / 1e9,
                     "frac": avg["total"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, "parts": avg},
        "stage_us": {k: v * 1e3 for k, v in stage.items()},
        "append_build": {"bytes": built_bytes, "s": t_build, "GB/s": built_bytes / max(t_build, 1e-9) / 1e9},
        "attnscore_reps": mass_res,
        "prune": prune_res,
        "lib_version": _lib.lib.brs_version(),
    })
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(w, layers[0][2], args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="infllm_gqa_decode_128k")
    ap.add_argument("--layers", type=int, default=0, help="layer memories to rotate over (0 = enough to exceed the cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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
    res = run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
