"""GPU parity of the offloaded memory (K/V in pinned host memory, a device
cache of blocks; InfLLM "method" offloading): a decode loop whose every
step's selection and output equal, bit for bit, those of the same loop on a
memory resident in device memory, with blocks copied only when missing or
grown and pages reused in least-recently-needed order."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import gpu_cases as C
from synth import WORKLOADS
from synth import inputs as I

pytestmark = pytest.mark.gpu

W = WORKLOADS


def pages_needed(w, N, lists):
    S = min(w.sinks, N)
    ws = max(N - w.window, S)
    nbt = -(-N // w.block)
    return -(-S // w.block) + (nbt - ws // w.block if ws < N else 0) + lists * w.k


@pytest.mark.parametrize("select", ["head", "group"])
def test_offload_decode_loop_matches_resident(select):
    import block_retrieval_sparse_amd as brs
    from block_retrieval_sparse_amd.pipeline import CachedStep, RetrievalStep

    w = W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=8192 + 37, window=512, sinks=64,
                                           k=8, planted_per_head=2)
    steps = 12
    cap = w.n_tokens + steps
    x = I.make_all(w, "cuda")
    kw = dict(dtype=torch.bfloat16, rep_mode=w.rep_mode, reps_per_block=w.reps_per_block, device="cuda")
    res = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, cap, w.block, **kw)
    off = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, cap, w.block, host=True, **kw)
    res.append(x["k"], x["v"])
    off.append(x["k"], x["v"])
    lists = w.n_kv_heads if select == "group" else w.n_q_heads
    # the bound for the longest memory of the loop: pages get evicted as selections change
    n_pages = pages_needed(w, cap, lists // w.n_kv_heads)
    cache = brs.BlockCache(off, n_pages)
    g = torch.Generator(device="cuda").manual_seed(7)
    prev_fetch = 0
    for t in range(steps):
        if t > 0:  # one new token per step
            kn = torch.randn((w.batch, w.n_kv_heads, 1, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
            vn = torch.randn((w.batch, w.n_kv_heads, 1, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
            res.append(kn, vn)
            off.append(kn, vn)
        q = torch.randn((w.batch, w.n_q_heads, 1, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
        if t == 0:
            q = x["q"]  # planted blocks for these queries
        qrep = q[:, :, -1, :].contiguous()
        a = RetrievalStep(res, w.n_q_heads, 1, w.k, w.sinks, w.window, select=select)
        a.run_separate(q, qrep)
        b = CachedStep(off, cache, w.n_q_heads, w.k, w.sinks, w.window, select=select)
        b.run(q, qrep)
        torch.cuda.synchronize()
        assert torch.equal(a.idx, b.idx), t
        assert torch.equal(a.out, b.out), (t, float((a.out - b.out).abs().max()))
        assert torch.equal(res.reps, off.reps), t
        total = int(cache.fetched.sum())
        assert total > prev_fetch or t > 0, t  # the first step copies every needed block
        prev_fetch = total
        if t == 0:
            wt = w.scaled(n_tokens=res.length)
            C.check_step(wt, res, dict(x, q=q), a, select=select)
    # the same step again: nothing new to copy
    before = int(cache.fetched.sum())
    b.run(q, qrep)
    torch.cuda.synchronize()
    assert int(cache.fetched.sum()) == before
    # every page still maps back to its block
    pob = cache.page_of_block.cpu().numpy()
    pblk = cache.page_block.cpu().numpy()
    for s in range(pob.shape[0]):
        for p, blk in enumerate(pblk[s]):
            if blk >= 0:
                assert pob[s, blk] == p, (s, p, blk)
        assert len(set(pblk[s][pblk[s] >= 0].tolist())) == int((pblk[s] >= 0).sum())


def test_offload_1m_token_memory_step():
    """A 1M-token memory (RetrievalAttention scale, one sequence, 8 kv heads)
    held in host memory: one step through the cache equals the resident
    step."""
    import block_retrieval_sparse_amd as brs
    from block_retrieval_sparse_amd.pipeline import CachedStep, RetrievalStep

    w = W["retrievalattn_gqa_decode_1m_b8"].scaled(batch=1)
    x = I.make_all(w, "cuda")
    kw = dict(dtype=torch.bfloat16, rep_mode=w.rep_mode, reps_per_block=w.reps_per_block, device="cuda")
    res = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, w.n_tokens, w.block, **kw)
    res.append(x["k"], x["v"])
    off = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, w.n_tokens, w.block, host=True, **kw)
    off.k.copy_(res.k.cpu())
    off.v.copy_(res.v.cpu())
    off.reps.copy_(res.reps)
    off.desc.length = res.length
    cache = brs.BlockCache(off, pages_needed(w, w.n_tokens, w.group))
    qrep = x["q"][:, :, -1, :].contiguous()
    a = RetrievalStep(res, w.n_q_heads, 1, w.k, w.sinks, w.window)
    a.run_separate(x["q"], qrep)
    b = CachedStep(off, cache, w.n_q_heads, w.k, w.sinks, w.window)
    b.run(x["q"], qrep)
    torch.cuda.synchronize()
    assert torch.equal(a.idx, b.idx)
    assert torch.equal(a.out, b.out)
    # the copied blocks are the per-kv-head unions of the selections
    idx = a.idx.cpu().numpy()
    want = sum(len(np.unique(idx[0, g * w.group:(g + 1) * w.group])) for g in range(w.n_kv_heads))
    assert int(cache.fetched.sum()) == want


CHUNK_CASES = {
    # chunked prefill on the matrix-core kernel, dot scores, one list per query head
    "prefill_dot": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=6000 + 11, block=64,
                                                      window=200, sinks=16, k=5, n_q=100, planted_per_head=0),
    # MemLong chunked prefill: cosine scores, one list per sequence, head dim 100 in rows of 104
    "prefill_cosine": W["memlong_chunk_prefill_80k"].scaled(n_q_heads=4, n_kv_heads=4, n_tokens=8 * 512 + 512),
    # head dim 64 (the kernel's 64-column contraction), two sequences, a short window
    "prefill_d64": W["retrievalattn_gqa_decode_1m_b8"].scaled(
        batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, rep_dim=64, n_tokens=4000 + 9, block=32, k=7, window=60,
        sinks=8, n_q=70, planted_per_head=0),
    # several queries on the slot kernels
    "decode_multi_q": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=6000, window=300, k=5,
                                                         n_q=3, planted_per_head=0),
}


@pytest.mark.parametrize("name,select", [(n, "head") for n in CHUNK_CASES] + [("prefill_dot", "group"),
                                                                             ("prefill_d64", "group"),
                                                                             ("decode_multi_q", "group")])
def test_offload_chunk_matches_resident(name, select):
    """A step of n_q > 1 queries (InfLLM "method": the memory units stay in
    host memory during chunked prefill too) over the cache equals the step
    on the resident memory, bit for bit: the prefill kernel reads its token
    rows through the page table as the slot kernels do."""
    import block_retrieval_sparse_amd as brs
    from block_retrieval_sparse_amd.pipeline import CachedStep, RetrievalStep

    w = CHUNK_CASES[name]
    res, x = C.load(w)
    rep_dtype = torch.bfloat16 if w.rep_mode == "embed" else I.torch_dtype(w)
    off = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, w.n_tokens, w.block, dtype=I.torch_dtype(w),
                       rep_mode=w.rep_mode, reps_per_block=w.reps_per_block, rep_dim=w.rep_dim, rep_dtype=rep_dtype,
                       row_stride=w.stride, device="cuda", host=True)
    given = x.get("given_reps", x.get("embeds"))
    off.append(x["k"], x["v"], given[:, :, :w.n_tokens // w.block] if given is not None else None)
    qrep = x["rq"] if w.rep_mode == "embed" else x["q"][:, :, -1, :].contiguous()
    a = RetrievalStep(res, w.n_q_heads, w.n_q, w.k, w.sinks, w.window, select=select)
    a.run_separate(x["q"], qrep)
    lists = 1 if (w.rep_mode == "embed" or select == "group") else w.group
    cache = brs.BlockCache(off, pages_needed(w, w.n_tokens, lists))
    b = CachedStep(off, cache, w.n_q_heads, w.k, w.sinks, w.window, select=select, n_q=w.n_q)
    b.run(x["q"], qrep)
    torch.cuda.synchronize()
    assert torch.equal(a.idx, b.idx)
    assert torch.equal(a.out, b.out), float((a.out - b.out).abs().max())
    assert int(cache.fetched.sum()) > 0
