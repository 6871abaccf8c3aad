"""GPU parity over a seeded sweep of shapes that no hand-picked case fixes.

Each case draws, from one fixed seed, a representative mode (mean, top-norm,
given, chunk embedding) and a storage type, a head dim (including dims that
are not powers of two), 1 or 2 kv heads with 1 to 8 query heads each, a block
size (including non-powers of two), a ragged token count, sinks and a window
(including none), k (sometimes above the number of candidates), one query,
two queries, or a chunk of 64 or more (the matrix-core prefill), and one
selection per query head or per kv head; a second set takes blocks of 256
to 512 tokens.  Every stage is compared with the
oracle under the same rules as the other parity tests: scores and selection
bit-exact, attention within the dtype's tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest

import gpu_cases as C
from synth import WORKLOADS

pytestmark = pytest.mark.gpu

W = WORKLOADS
KINDS = ("mean", "topnorm", "given", "embed", "f32")
BASE = {"mean": "retrievalattn_gqa_decode_1m_b8", "topnorm": "infllm_gqa_decode_128k",
        "given": "landmark_decode_32k", "embed": "memlong_chunk_prefill_80k", "f32": "tiny_decode"}


def sweep_case(i: int, seed: int = 20241203):
    rng = np.random.default_rng([seed, i])
    kind = KINDS[i % len(KINDS)]
    bf16 = kind != "f32"
    d = int(rng.choice([32, 48, 64, 80, 96, 100, 112, 128] if bf16 else [16, 32, 48, 64]))
    stride = -(-d // 8) * 8 if bf16 else d
    if kind == "embed":
        hkv, G = int(rng.choice([2, 4])), 1
    else:
        hkv, G = int(rng.choice([1, 2])), int(rng.choice([1, 2, 4, 8]))
    block = int(rng.choice([16, 32, 50, 64, 100, 128]))
    nb = int(rng.integers(12, 48))
    n_tokens = nb * block + int(rng.integers(0, block))
    u = rng.random()
    n_q = int(rng.choice([64, 70, 100])) if (bf16 and u < 0.4) else (2 if u < 0.6 else 1)
    window = int(rng.choice([0, block // 2, 2 * block, 3 * block + 5]))
    sinks = int(rng.choice([0, 1, 7, block]))
    k = nb + 3 if rng.random() < 0.15 else int(rng.integers(1, 24))
    R = int(rng.integers(1, 5)) if kind == "topnorm" else 1
    rep_dim = int(rng.choice([64, 128, 256])) if kind == "embed" else d
    select = "group" if (kind != "embed" and G > 1 and rng.random() < 0.4) else "head"
    w = W[BASE[kind]].scaled(
        name=f"sweep{i}", batch=1 + int(rng.random() < 0.3), n_q_heads=hkv * G, n_kv_heads=hkv, head_dim=d,
        row_stride=stride, n_tokens=n_tokens, block=block, reps_per_block=R, rep_dim=rep_dim, k=k, window=window,
        sinks=sinks, n_q=n_q, planted_per_head=0, ood_offset=float(rng.choice([0.0, 2.0])), seed=7000 + i)
    return w, select


CASES = [sweep_case(i) for i in range(25)]


def sweep_case_long_blocks(i: int, seed: int = 20261203):
    """Blocks of 256 to 512 tokens, mostly with query chunks: the stream's
    first segment (sinks, a selected block or the window) can then cover the
    prefill kernel's first four stages, which it requests before building the
    segments; k up to the candidate count and beyond."""
    rng = np.random.default_rng([seed, i])
    kind = ("mean", "topnorm", "given", "embed")[i % 4]
    d = int(rng.choice([64, 96, 100, 128]))
    stride = -(-d // 8) * 8
    hkv, G = (int(rng.choice([2, 4])), 1) if kind == "embed" else (int(rng.choice([1, 2])), int(rng.choice([1, 2, 4])))
    block = int(rng.choice([256, 300, 512]))
    nb = int(rng.integers(6, 24))
    n_tokens = nb * block + int(rng.integers(0, block))
    n_q = int(rng.choice([64, 96, 130])) if rng.random() < 0.8 else 1
    window = int(rng.choice([0, 100, block, 2 * block + 17]))
    sinks = int(rng.choice([0, 0, 64, 300]))
    k = nb + 2 if rng.random() < 0.2 else int(rng.integers(1, 8))
    R = int(rng.integers(1, 5)) if kind == "topnorm" else 1
    rep_dim = int(rng.choice([64, 256])) if kind == "embed" else d
    select = "group" if (kind != "embed" and G > 1 and rng.random() < 0.4) else "head"
    w = W[BASE[kind]].scaled(
        name=f"sweepL{i}", batch=1 + int(rng.random() < 0.3), n_q_heads=hkv * G, n_kv_heads=hkv, head_dim=d,
        row_stride=stride, n_tokens=n_tokens, block=block, reps_per_block=R, rep_dim=rep_dim, k=k, window=window,
        sinks=sinks, n_q=n_q, planted_per_head=0, ood_offset=float(rng.choice([0.0, 2.0])), seed=9000 + i)
    return w, select


CASES += [sweep_case_long_blocks(i) for i in range(12)]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_sweep_case(i):
    from block_retrieval_sparse_amd.pipeline import RetrievalStep

    w, select = CASES[i]
    print(f"case {i}: {w.rep_mode} {w.dtype} d={w.head_dim} hq={w.n_q_heads} hkv={w.n_kv_heads} B={w.block} "
          f"N={w.n_tokens} S={w.sinks} W={w.window} k={w.k} n_q={w.n_q} R={w.reps_per_block} select={select}",
          flush=True)
    mem, x = C.load(w, pieces=2)
    step = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k, w.sinks, w.window, select=select)
    qrep = x["rq"] if w.rep_mode == "embed" else x["q"][:, :, -1, :].contiguous()
    step.run(x["q"], qrep)
    C.check_step(w, mem, x, step, select=select)
