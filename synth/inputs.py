"""Seeded synthetic inputs for the block-retrieval workloads.

Both sides of every parity check take their inputs from here: the HIP path
receives the device tensors, the oracle receives host copies of the very same
tensors. This module draws random numbers and lays them out; it computes none
of the method's arithmetic (no representatives, scores, selection or
attention).

Recipe
------
* Every tensor is drawn in float32 from ``torch.randn`` with a generator
  seeded per unit ``(workload seed, tensor id, batch, head, token chunk)``;
  bfloat16 tensors are the float32 draws rounded to nearest-even by torch.
* K and V are drawn in units of ``GEN_CHUNK`` tokens per (batch, kv head), so
  any token range can be regenerated on its own (the 1M-token workload is
  never held whole on the host).
* Queries are drawn first.  Planted blocks (InfLLM-style needle check): for
  every query head h, ``planted_per_head`` distinct blocks of kv head g(h),
  disjoint across the heads of one group and lying wholly outside the sinks
  and the window, get keys ``planted_scale * q_h + N(0, I)`` on every token.
* Out-of-distribution queries (RetrievalAttention-style):
  ``q = ood_offset * u + N(0, I)`` with one random unit vector u shared by
  every batch row and head.
* Landmark keys (``given``) are independent N(0, I) vectors, one per block.
* Chunk embeddings (``embed``, MemLong-style, d_ret = 768) are N(0, I)
  vectors normalised in float32 and then rounded to bfloat16; the last one
  belongs to the current chunk and is also the query embedding.

The generator device is a parameter: on a GPU machine the tensors are drawn
there (torch's device generator), on a CPU-only host they are drawn on the
CPU.  The two streams differ, which is fine: each check feeds one draw to both
sides.
"""
from __future__ import annotations

import hashlib

import torch

from .workloads import Workload

GEN_CHUNK = 65536  # tokens per generation unit

T_K, T_V, T_Q, T_PLANT_POS, T_PLANT_NOISE, T_LANDMARK, T_EMBED, T_OOD_DIR = range(8)


def unit_seed(base: int, *parts: int) -> int:
    h = hashlib.sha256(("/".join(str(p) for p in (base,) + parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, device, seed: int) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def make_queries(w: Workload, device) -> torch.Tensor:
    """q of shape [batch][n_q_heads][n_q][head_dim] in the workload dtype."""
    dt = torch_dtype(w)
    q = torch.empty((w.batch, w.n_q_heads, w.n_q, w.head_dim), dtype=dt, device=device)
    u = None
    if w.ood_offset:
        u = randn((w.head_dim,), device, unit_seed(w.seed, T_OOD_DIR))
        u = u / torch.linalg.vector_norm(u)
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            x = randn((w.n_q, w.head_dim), device, unit_seed(w.seed, T_Q, b, h))
            if u is not None:
                x = x + w.ood_offset * u
            q[b, h] = x.to(dt)
    return q


def planted_blocks(w: Workload, device="cpu") -> dict:
    """{(b, h): [block, ...]} for the planted workload, else {}.

    Blocks are drawn from those lying wholly outside the first ``sinks``
    tokens and the last ``window`` tokens.
    """
    if not w.planted_per_head:
        return {}
    first = -(-w.sinks // w.block)
    last = (w.n_tokens - w.window) // w.block  # exclusive
    pool = last - first
    need = w.planted_per_head * w.group
    if pool < need:
        raise ValueError(f"{w.name}: {pool} plantable blocks < {need}")
    out = {}
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            perm = torch.randperm(pool, generator=_gen("cpu", unit_seed(w.seed, T_PLANT_POS, b, g)))
            chosen = (perm[:need] + first).tolist()
            for j in range(w.group):
                h = g * w.group + j
                out[(b, h)] = sorted(chosen[j * w.planted_per_head:(j + 1) * w.planted_per_head])
    return out


def make_kv(w: Workload, device, q: torch.Tensor | None = None, t0: int = 0, t1: int | None = None):
    """K, V for tokens [t0, t1) of every (batch, kv head): [batch][n_kv][t1-t0][head_dim].

    ``q`` (from :func:`make_queries`) is required when the workload plants
    blocks, since planted keys are built from it.
    """
    t1 = w.n_tokens if t1 is None else t1
    n = t1 - t0
    dt = torch_dtype(w)
    K = torch.empty((w.batch, w.n_kv_heads, n, w.head_dim), dtype=dt, device=device)
    V = torch.empty_like(K)
    c0, c1 = t0 // GEN_CHUNK, -(-t1 // GEN_CHUNK)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            for c in range(c0, c1):
                u0 = c * GEN_CHUNK
                u1 = min(u0 + GEN_CHUNK, w.n_tokens)
                a, z = max(u0, t0), min(u1, t1)
                for T, tid in ((K, T_K), (V, T_V)):
                    x = randn((u1 - u0, w.head_dim), device, unit_seed(w.seed, tid, b, g, c))
                    T[b, g, a - t0:z - t0] = x[a - u0:z - u0].to(dt)
    plants = planted_blocks(w)
    if plants:
        if q is None:
            raise ValueError("planted workload: pass q")
        for (b, h), blocks in plants.items():
            g = h // w.group
            qh = q[b, h, -1].to(torch.float32)
            for blk in blocks:
                a, z = max(blk * w.block, t0), min((blk + 1) * w.block, t1)
                if a >= z:
                    continue
                noise = randn((w.block, w.head_dim), device, unit_seed(w.seed, T_PLANT_NOISE, b, h, blk))
                keys = w.planted_scale * qh[None, :] + noise
                K[b, g, a - t0:z - t0] = keys[a - blk * w.block:z - blk * w.block].to(dt)
    return K, V


def make_given_reps(w: Workload, device, n_blocks: int | None = None) -> torch.Tensor:
    """Landmark keys: [batch][n_kv][n_blocks][reps_per_block][head_dim], N(0, I)."""
    nb = w.n_blocks if n_blocks is None else n_blocks
    dt = torch_dtype(w)
    out = torch.empty((w.batch, w.n_kv_heads, nb, w.reps_per_block, w.head_dim), dtype=dt, device=device)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            x = randn((nb, w.reps_per_block, w.head_dim), device, unit_seed(w.seed, T_LANDMARK, b, g))
            out[b, g] = x.to(dt)
    return out


def make_embeddings(w: Workload, device, n_blocks: int | None = None) -> torch.Tensor:
    """Chunk embeddings: [batch][1][n_blocks][1][rep_dim] bf16, unit norm before rounding.

    The last one is the current chunk's embedding (its query embedding).
    """
    nb = w.n_blocks if n_blocks is None else n_blocks
    out = torch.empty((w.batch, 1, nb, 1, w.rep_dim), dtype=torch.bfloat16, device=device)
    for b in range(w.batch):
        x = randn((nb, w.rep_dim), device, unit_seed(w.seed, T_EMBED, b))
        x = x / torch.linalg.vector_norm(x, dim=1, keepdim=True)
        out[b, 0, :, 0, :] = x.to(torch.bfloat16)
    return out


def make_all(w: Workload, device) -> dict:
    """Everything one step of workload ``w`` needs, compact layout, on ``device``."""
    q = make_queries(w, device)
    K, V = make_kv(w, device, q=q)
    d = {"q": q, "k": K, "v": V, "planted": planted_blocks(w)}
    if w.rep_mode == "given":
        d["given_reps"] = make_given_reps(w, device)
    if w.rep_mode == "embed":
        e = make_embeddings(w, device)
        d["embeds"] = e
        d["rq"] = e[:, :, -1, 0, :].contiguous()
    return d
