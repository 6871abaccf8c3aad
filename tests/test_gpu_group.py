"""GPU parity of the shared per-group selection (grouped-query attention):
one selection per kv head, ranked by the maximum of the group's query heads'
dot-max scores, attended by every head of the group -- decode (in the
attention kernel and through the separate calls) and the matrix-core chunked
prefill, against the oracle's ``scores_group_max`` / ``step(select="group")``.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_cases as C
from synth import WORKLOADS

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    "infllm": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=8192 + 37, window=512,
                                                  k=8, planted_per_head=2),
    "gqa8": W["infllm_gqa_decode_128k"].scaled(n_q_heads=16, n_kv_heads=2, n_tokens=4096 + 100, window=256,
                                                sinks=64, k=6, planted_per_head=0),
    "retrieval_mean": W["retrievalattn_gqa_decode_1m_b8"].scaled(batch=2, n_q_heads=8, n_kv_heads=2,
                                                                  n_tokens=16384, k=40),
    "multi_q": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=6000, window=300, k=5,
                                                   n_q=3, planted_per_head=0),
    "landmark_given": W["landmark_decode_32k"].scaled(n_q_heads=8, n_kv_heads=4, n_tokens=3018, k=6),
    # chunk of queries on the matrix-core prefill kernel: the chunk's last query represents each head
    "prefill_gqa": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=6000 + 11, block=64,
                                                       window=200, sinks=16, k=5, n_q=100, planted_per_head=0),
}


def run_group(mem, w, x, separate=False):
    from block_retrieval_sparse_amd.pipeline import RetrievalStep

    step = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k, w.sinks, w.window, select="group")
    qrep = x["q"][:, :, -1, :].contiguous()
    if separate:
        step.run_separate(x["q"], qrep)
    else:
        step.run(x["q"], qrep)
    torch.cuda.synchronize()
    return step


@pytest.mark.parametrize("name", list(CASES))
def test_group_step(name):
    w = CASES[name]
    mem, x = C.load(w)
    step = run_group(mem, w, x)
    assert tuple(step.idx.shape) == (w.batch, w.n_kv_heads, w.k)
    res = C.check_step(w, mem, x, step, select="group")
    print(f"{name} (group selection): max |err| {res['max_abs_err']:.3g}")
    if w.planted_per_head and w.k >= w.planted_per_head * w.group:
        idx = step.idx.cpu().numpy()
        for (b, h), blocks in x["planted"].items():
            assert set(blocks) <= set(idx[b, h // w.group].tolist()), (b, h)


@pytest.mark.parametrize("name", ["infllm", "gqa8", "prefill_gqa"])
def test_group_one_call_matches_three_calls(name):
    """brs_retrieval_step with one list per kv head against brs_score_blocks_group,
    brs_select_topk and brs_retrieval_attention (idx_heads = n_kv_heads): the
    same bits."""
    w = CASES[name]
    mem, x = C.load(w)
    one = run_group(mem, w, x)
    three = run_group(mem, w, x, separate=True)
    lo, hi = one.lo, one.hi
    assert torch.equal(one.idx, three.idx)
    assert torch.equal(one.scores[:, :, lo:hi], three.scores[:, :, lo:hi])
    assert torch.equal(one.out, three.out)


def test_group_full_size_infllm_128k():
    """The 128K grouped-query workload (32 query / 8 kv heads, 4 representatives
    per block, k = 32) with one selection per kv head: every head checked; the
    32 blocks planted for a group's four heads are exactly its selection."""
    w = W["infllm_gqa_decode_128k"]
    mem, x = C.load(w)
    step = run_group(mem, w, x)
    res = C.check_step(w, mem, x, step, select="group")
    idx = step.idx.cpu().numpy()
    for g in range(w.n_kv_heads):
        planted = set()
        for h in range(g * w.group, (g + 1) * w.group):
            planted |= set(x["planted"][(0, h)])
        assert set(idx[0, g].tolist()) == planted, g
    print(f"128K group selection: max |err| {res['max_abs_err']:.3g}")
