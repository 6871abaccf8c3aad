"""GPU parity for MemLong's retrieval counters and pruning (section 2.3.2,
dynamic memory update), through the C ABI against the CPU oracle: the
counts are exact integers, the plan (every block's new index) is bit-exact,
and the pruned memory's K, V, representatives and counts are bit-exact
copies of the kept blocks, with the partial tail behind them.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_cases as C
import oracle.brs_oracle as O

pytestmark = pytest.mark.gpu


def _memory(dtype, rep_mode, batch, hkv, d, B, R, n_tokens, capacity, seed):
    import block_retrieval_sparse_amd as brs

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    embed = rep_mode == "embed"
    mem = brs.KVMemory(batch, hkv, d, capacity, B, dtype=tdt, rep_mode=rep_mode, reps_per_block=R,
                       rep_dim=64 if embed else d, rep_dtype=torch.bfloat16 if embed else tdt)
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = torch.randn((batch, hkv, n_tokens, d), generator=g).to(tdt).cuda()
    v = torch.randn((batch, hkv, n_tokens, d), generator=g).to(tdt).cuda()
    reps = None
    if embed:
        reps = torch.randn((batch, 1, n_tokens // B, 1, 64), generator=g).to(torch.bfloat16).cuda()
    mem.append(k, v, reps)
    return mem, g


def test_count_hits_accumulates_valid_entries():
    mem, g = _memory("bf16", "mean", 2, 2, 64, 16, 1, 16 * 50 + 7, 16 * 64, 5)
    nb = mem.n_blocks
    hits = mem.new_hits()
    want = np.zeros((2, mem.blocks_stride), dtype=np.int64)
    for _ in range(3):
        idx = torch.randint(-2, nb + 3, (2, 4, 9), generator=g, dtype=torch.int32)
        mem.count_hits(idx.cuda(), hits)
        for b in range(2):
            for h in range(4):
                want[b, :nb] = O.count_hits(want[b, :nb], idx[b, h].numpy(), nb)
    torch.cuda.synchronize()
    assert np.array_equal(hits.cpu().numpy(), want)


CASES = [
    # dtype, rep_mode, batch, kv heads, d, B, R, tokens, capacity
    ("bf16", "topnorm", 1, 2, 128, 32, 4, 32 * 200 + 13, 32 * 210),
    ("f32", "mean", 2, 1, 64, 16, 1, 16 * 97, 16 * 100),
    ("bf16", "embed", 1, 4, 64, 64, 1, 64 * 40 + 63, 64 * 41),
    ("bf16", "attnscore", 1, 2, 128, 8, 2, 8 * 3000 + 5, 8 * 3001),  # thousands of middle blocks
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-nb{c[7] // c[5]}" for c in CASES])
def test_prune_matches_oracle(case):
    dtype, rep_mode, batch, hkv, d, B, R, N, cap = case
    mem, g = _memory(dtype, rep_mode, batch, hkv, d, B, R, N, cap, 11)
    if rep_mode == "attnscore":
        mem.reps_from_mass(mem.new_mass(), 0, mem.n_blocks)
    nb = mem.n_blocks
    hits = torch.zeros((batch, mem.blocks_stride), dtype=torch.int32)
    hits[:, :nb] = torch.randint(0, 3, (batch, nb), generator=g, dtype=torch.int32)  # many ties
    hits = hits.cuda()
    dst = mem.like()
    dst_hits = torch.full_like(hits, -7)
    plan = mem.prune_into(hits, dst, dst_hits)
    torch.cuda.synchronize()
    hsum = hits.cpu().numpy()[:, :nb].sum(axis=0)
    want = O.prune_plan(N, B, cap, hsum)
    got = plan.cpu().numpy()[:nb]
    assert np.array_equal(got, want)
    kept = int((want >= 0).sum())
    assert 0 < kept < nb
    assert dst.length == kept * B + (N - nb * B)
    n2 = dst.length
    for b in range(batch):
        for h in range(hkv):
            for name in ("k", "v"):
                src = C.host(getattr(mem, name)[b, h, :N])
                assert np.array_equal(C.host(getattr(dst, name)[b, h, :n2]), O.compact(src, want, B, N)), (b, h)
    old = [i for i in range(nb) if want[i] >= 0]
    assert torch.equal(dst.reps[:, :, :kept], mem.reps[:, :, old])
    assert torch.equal(dst_hits[:, :kept], hits[:, old])


def test_prune_small_and_saturated():
    """Fewer than ten blocks (no tenth to drop or keep) and a capacity that fits everything: the plan is the
    identity.  Counts that fall with age: the newest middle blocks (fewest hits) are the ones evicted."""
    # identity: 7 blocks and a tail, half the capacity holds them all
    mem, g = _memory("bf16", "mean", 1, 2, 64, 16, 1, 16 * 7 + 3, 16 * 20, 3)
    hits = mem.new_hits()
    dst = mem.like()
    plan = mem.prune_into(hits, dst)
    torch.cuda.synchronize()
    assert plan.cpu().numpy()[:7].tolist() == list(range(7))
    assert dst.length == mem.length
    assert torch.equal(dst.k[:, :, :mem.length], mem.k[:, :, :mem.length])
    # 100 blocks, capacity 2000 tokens: half holds 62 blocks, so 52 of the 80 middle blocks stay
    mem2, g2 = _memory("bf16", "mean", 1, 1, 64, 16, 1, 16 * 100, 16 * 125, 4)
    hits2 = mem2.new_hits()
    hits2[0, :100] = torch.arange(100, 0, -1, dtype=torch.int32, device=hits2.device)  # older = more hits
    dst2 = mem2.like()
    plan2 = mem2.prune_into(hits2, dst2).cpu().numpy()[:100]
    torch.cuda.synchronize()
    want = O.prune_plan(1600, 16, 2000, hits2.cpu().numpy()[0, :100])
    assert np.array_equal(plan2, want)
    assert (plan2[:10] == -1).all() and (plan2[10:62] >= 0).all() and (plan2[62:90] == -1).all()


def test_count_hits_broadcast_lists():
    """One selection list per sequence (idx_heads = 1)."""
    mem, g = _memory("f32", "mean", 3, 1, 64, 16, 1, 16 * 30, 16 * 32, 6)
    hits = mem.new_hits()
    idx = torch.tensor([[[0, 5, 5, 29, -1]], [[30, 1, 1, 1, 2]], [[7, 7, 7, 7, 7]]], dtype=torch.int32)
    mem.count_hits(idx.cuda(), hits)
    torch.cuda.synchronize()
    got = hits.cpu().numpy()[:, :30]
    assert got[0, 0] == 1 and got[0, 5] == 2 and got[0, 29] == 1 and got[0].sum() == 4
    assert got[1, 1] == 3 and got[1, 2] == 1 and got[1].sum() == 4  # block 30 is not complete
    assert got[2, 7] == 5 and got[2].sum() == 5
