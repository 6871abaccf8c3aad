"""Helpers for the GPU parity tests: load a synthetic workload into the HIP
library, run its stages, and compare each stage with the CPU oracle.

Comparison rules (block-retrieval hot path):
* representatives and scores: bit-exact (both sides sum exact products in
  float64 and round once);
* top-k indices: bit-exact, except where the oracle's k-th and (k+1)-th
  scores are within 1e-6 relative -- then blocks inside that tie band may
  differ, everything outside it must match;
* attention: the oracle is evaluated on the GPU's own selection, and must
  agree within 1e-5 absolute (float32 inputs) or 2e-3 absolute (bfloat16
  inputs, float32 accumulation).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.brs_oracle as O
from synth import inputs as I
from synth.workloads import Workload

TOL = {"f32": 1e-5, "bf16": 2e-3}


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def load(w: Workload, device="cuda", pieces: int = 1, capacity: int | None = None, x: dict | None = None):
    """Generate workload ``w`` (or take its inputs ``x``) and append it into a
    fresh KVMemory in ``pieces`` appends."""
    import block_retrieval_sparse_amd as brs

    if x is None:
        x = I.make_all(w, device)
    rep_dtype = torch.bfloat16 if w.rep_mode == "embed" else I.torch_dtype(w)
    mem = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, capacity or w.n_tokens, w.block,
                       dtype=I.torch_dtype(w), rep_mode=w.rep_mode, reps_per_block=w.reps_per_block,
                       rep_dim=w.rep_dim, rep_dtype=rep_dtype, row_stride=w.stride, device=device)
    given = x.get("given_reps", x.get("embeds"))
    cuts = sorted(set([0, w.n_tokens] + [int(w.n_tokens * (i + 1) / pieces) + i * 7 for i in range(pieces - 1)]))
    cuts = [c for c in cuts if 0 <= c <= w.n_tokens]
    for a, z in zip(cuts[:-1], cuts[1:]):
        b0, b1 = a // w.block, z // w.block
        rn = given[:, :, b0:b1] if (given is not None and b1 > b0) else None
        mem.append(x["k"][:, :, a:z], x["v"][:, :, a:z], rn)
    return mem, x


def oracle_reps(w: Workload, x: dict, pairs=None) -> dict:
    """O1 per (batch, rep head) on host copies of the generated inputs."""
    out = {}
    nb = w.n_blocks
    if w.rep_mode in ("given", "embed"):
        src = host(x["given_reps"] if w.rep_mode == "given" else x["embeds"])
        for b in range(w.batch):
            for g in range(src.shape[1]):
                out[(b, g)] = src[b, g, :nb]
        return out
    want = pairs if pairs is not None else [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    for (b, g) in want:
        K = host(x["k"][b, g])
        out[(b, g)] = O.build_reps(K, w.rep_mode, w.block, w.reps_per_block, w.dtype)
    return out


def check_reps(w: Workload, mem, ref: dict) -> None:
    nb = w.n_blocks
    got = host(mem.reps)
    for (b, g), r in ref.items():
        assert np.array_equal(got[b, g, :nb], r), f"reps differ at batch {b} head {g}"


def check_idx(gidx: np.ndarray, oidx: np.ndarray, oscores: np.ndarray, k: int, what: str) -> None:
    if np.array_equal(gidx, oidx):
        return
    valid = oidx[oidx >= 0]
    assert len(valid) == k, f"{what}: selection differs: gpu {gidx} oracle {oidx}"
    a = float(oscores[oidx[k - 1]])
    band = set(np.flatnonzero(np.abs(oscores - a) / np.maximum(np.maximum(np.abs(oscores), abs(a)), 1e-30) < 1e-6))
    for j in range(k):
        if gidx[j] != oidx[j]:
            assert int(oidx[j]) in band and int(gidx[j]) in band, (
                f"{what}: slot {j}: gpu {gidx[j]} oracle {oidx[j]} outside the 1e-6 tie band")


def check_step(w: Workload, mem, x: dict, step, pairs=None, query_rows=None, check_scores=True,
               select: str = "head") -> dict:
    """Compare scores, selection and attention of an executed RetrievalStep with
    the oracle on the (batch, query head) ``pairs`` (default: all).  With
    ``select="group"`` the selection is one per kv head (group scores)."""
    torch.cuda.synchronize()
    N = mem.length
    lo, hi = O.eligible_range(N, w.block, w.sinks, w.window)
    assert (lo, hi) == (step.lo, step.hi), ((lo, hi), (step.lo, step.hi))
    G = w.group
    pairs = pairs if pairs is not None else [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)]
    need = sorted({(b, 0 if w.rep_mode == "embed" else h // G) for (b, h) in pairs})
    reps = oracle_reps(w, x, pairs=need)
    gscores, gidx, gout = host(step.scores), step.idx.cpu().numpy(), step.out.detach().cpu().numpy()
    q = host(x["q"])
    rq = host(x["rq"]).reshape(w.batch, -1) if w.rep_mode == "embed" else None
    scale = step.scale
    worst = 0.0
    done_sel = set()
    for (b, h) in pairs:
        g = O.kv_head_of(h, w.n_q_heads, w.n_kv_heads)
        sh = 0 if w.rep_mode == "embed" else (g if select == "group" else h)
        key = (b, sh)
        if key not in done_sel:
            done_sel.add(key)
            if w.rep_mode == "embed":
                s = O.scores_cosine(rq[b], reps[(b, 0)][lo:hi, 0, :])
            elif select == "group":
                s = O.scores_group_max(q[b, g * G:(g + 1) * G, -1], reps[(b, g)][lo:hi])
            else:
                s = O.scores_dot_max(q[b, h, -1], reps[(b, g)][lo:hi])
            full = np.full(gscores.shape[2], np.nan, dtype=np.float32)
            full[lo:hi] = s
            if check_scores and hi > lo:
                gs = gscores[b, sh, lo:hi].astype(np.float32)
                bad = np.flatnonzero(gs.view(np.uint32) != s.view(np.uint32))
                assert bad.size == 0, f"scores differ at batch {b} head {sh}: blocks {bad[:8] + lo}"
            oidx, _ = O.select_topk(full, lo, hi, w.k)
            check_idx(gidx[b, sh], oidx, full, w.k, f"batch {b} head {sh}")
        T = O.attended_mask(N, w.block, w.sinks, w.window, gidx[b, sh])
        Kh, Vh = host(x["k"][b, g]), host(x["v"][b, g])   # the generator's tensors, not the memory
        rows = list(range(w.n_q)) if query_rows is None else query_rows
        Qsel = q[b, h]
        ref_all = None
        if query_rows is None:
            ref_all = O.attention(Qsel, Kh, Vh, T, scale)
        for j in rows:
            if ref_all is not None:
                ref = ref_all[j]
            else:
                # query j alone sits at p = N - n_q + j: a one-query call on the first p + 1 tokens
                p = N - w.n_q + j
                ref = O.attention(Qsel[j:j + 1], Kh[:p + 1], Vh[:p + 1], T[:p + 1], scale)[0]
            err = float(np.max(np.abs(gout[b, h, j] - ref)))
            worst = max(worst, err)
            assert err <= TOL[w.dtype], f"attention differs at batch {b} head {h} query {j}: {err:.3g}"
    return {"max_abs_err": worst}


def scale_of(w: Workload) -> float:
    return 1.0 / math.sqrt(w.head_dim)
