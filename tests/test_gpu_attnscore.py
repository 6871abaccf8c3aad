"""GPU parity for attention-score representatives (InfLLM "method": a memory
unit is represented by the tokens that received the most attention while in
the local window), through the C ABI against the CPU oracle.

* lse: each query's log-sum-exp from the attention call, against
  ``attention_lse`` on the GPU's own selection (decode and chunked prefill);
* window mass: one ``brs_window_mass`` call against ``window_mass``;
* representatives from a given mass: bit-exact against ``reps_attnscore``
  (ties planted);
* a decode loop (append, step, accumulate, refresh): the accumulated mass
  against the oracle's, and every built block's representatives against
  ``reps_attnscore`` of the GPU's mass.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_cases as C
import oracle.brs_oracle as O
from synth import WORKLOADS

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    "decode_gqa": W["infllm_gqa_decode_128k"].scaled(rep_mode="attnscore", n_q_heads=8, n_kv_heads=2,
                                                     n_tokens=6000 + 37, window=512, sinks=16, k=8,
                                                     planted_per_head=0),
    "prefill_gqa": W["infllm_gqa_decode_128k"].scaled(rep_mode="attnscore", n_q_heads=8, n_kv_heads=2,
                                                      n_tokens=5000 + 11, block=64, window=300, sinks=16, k=5,
                                                      n_q=100, planted_per_head=0),
    "decode_f32": W["tiny_decode"].scaled(rep_mode="attnscore", reps_per_block=3, n_q_heads=4, n_kv_heads=2,
                                          n_tokens=3000, block=50, k=5, window=200, sinks=10),
    # a window shorter than the query chunk (early queries see none of it beyond their own position)
    "prefill_short_window": W["retrievalattn_gqa_decode_1m_b8"].scaled(
        rep_mode="attnscore", reps_per_block=2, batch=2, n_q_heads=4, n_kv_heads=4, head_dim=64, rep_dim=64,
        n_tokens=4000, block=32, k=10, window=40, n_q=150),
    # the window covers the whole memory (no candidates, k = 0 path)
    "window_all": W["tiny_decode"].scaled(rep_mode="attnscore", reps_per_block=2, n_q_heads=2, n_kv_heads=1,
                                          n_tokens=700, block=64, k=0, window=4096, sinks=0),
}
MASS_RTOL, MASS_ATOL = 1e-4, 1e-6


def _step(mem, w, x, want_lse=True):
    from block_retrieval_sparse_amd.pipeline import RetrievalStep

    step = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k, w.sinks, w.window, want_lse=want_lse)
    step.run(x["q"], x["q"][:, :, -1, :].contiguous())
    return step


def _oracle_sets(w, step):
    """The GPU's selection turned into each (batch, head)'s attended set."""
    idx = step.idx.cpu().numpy() if w.k else np.full((w.batch, w.n_q_heads, 1), -1)
    return {(b, h): O.attended_mask(w.n_tokens, w.block, w.sinks, w.window, idx[b, h])
            for b in range(w.batch) for h in range(w.n_q_heads)}


@pytest.mark.parametrize("name", list(CASES))
def test_lse_and_window_mass(name):
    w = CASES[name]
    from block_retrieval_sparse_amd.pipeline import AttnScoreMemory

    mem, x = C.load(w)
    AS = AttnScoreMemory(mem, w.sinks, w.window)
    AS.refresh()  # representatives of the initial candidates (mass still zero: lowest tokens)
    step = _step(mem, w, x)
    AS.accumulate(x["q"], step.lse)
    torch.cuda.synchronize()
    T = _oracle_sets(w, step)
    q, lse, mass = C.host(x["q"]), step.lse.cpu().numpy(), AS.mass.cpu().numpy()
    G = w.group
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            K = C.host(x["k"][b, g])
            for h in range(g * G, (g + 1) * G):
                want = O.attention_lse(q[b, h], K, T[(b, h)], step.scale)
                assert np.allclose(lse[b, h], want, rtol=1e-5, atol=1e-4), (b, h, lse[b, h][:4], want[:4])
            want_m = np.zeros(w.n_tokens)
            for h in range(g * G, (g + 1) * G):
                want_m += O.window_mass(q[b, h][None], K, T[(b, h)], step.scale, w.window)
            got = mass[b, g, : w.n_tokens]
            assert np.allclose(got, want_m, rtol=MASS_RTOL, atol=MASS_ATOL), \
                (b, g, np.abs(got - want_m).max())
            assert (got[: max(w.n_tokens - w.window, 0)] == 0).all()
    # mass of a decode call: each head's window weights sum to at most 1
    if w.n_q == 1:
        tot = mass.sum(axis=2)
        assert (tot <= G * (1 + 1e-5)).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reps_from_given_mass_with_ties(dtype):
    import block_retrieval_sparse_amd as brs

    B, R, nb, d, Hkv = 64, 4, 40, 128, 2
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mem = brs.KVMemory(1, Hkv, d, nb * B, B, dtype=tdt, rep_mode="attnscore", reps_per_block=R)
    g = torch.Generator(device="cpu").manual_seed(1234)
    K = torch.randn((1, Hkv, nb * B, d), generator=g).to(tdt)
    mem.append(K.cuda(), K.cuda())
    mass = torch.randint(0, 5, (1, Hkv, nb * B), generator=g).to(torch.float32)  # heavy ties
    mass[0, 0, 5 * B + 7] = 1e9    # one token far above its block
    mass[0, 1, 9 * B:10 * B] = 2.5  # a whole block tied
    mem.reps_from_mass(mass.cuda(), 3, 31)
    torch.cuda.synchronize()
    got = C.host(mem.reps[0, :, 3:31])
    for h in range(Hkv):
        want = O.reps_attnscore(C.host(K[0, h]), mass[0, h].double().numpy(), B, R, list(range(3, 31)))
        assert np.array_equal(got[h], want), h
    assert not mem.reps[0, :, :3].any() and not mem.reps[0, :, 31:].any()


def test_decode_loop_accumulates_and_builds():
    """Append, step, accumulate, refresh, 48 times: the mass against the
    oracle's replay of the same steps (on the GPU's selections), and every
    built block's representatives against ``reps_attnscore`` of the GPU's mass."""
    from block_retrieval_sparse_amd.pipeline import AttnScoreMemory, RetrievalStep

    w = CASES["decode_gqa"].scaled(n_tokens=3000, window=256, block=32, k=6)
    steps = 48
    cap = w.n_tokens + steps
    mem, x = C.load(w, capacity=cap)
    gen = torch.Generator(device="cpu").manual_seed(77)
    dt = mem.k.dtype
    AS = AttnScoreMemory(mem, w.sinks, w.window)
    built = [AS.refresh()]
    at_build = {}  # block range -> the GPU mass when it was built
    K_all = C.host(x["k"])
    oracle_mass = np.zeros((w.batch, w.n_kv_heads, cap))
    G = w.group
    for s in range(steps):
        kn = torch.randn((w.batch, w.n_kv_heads, 1, w.head_dim), generator=gen).to(dt)
        vn = torch.randn((w.batch, w.n_kv_heads, 1, w.head_dim), generator=gen).to(dt)
        q = torch.randn((w.batch, w.n_q_heads, 1, w.head_dim), generator=gen).to(dt).cuda()
        mem.append(kn.cuda(), vn.cuda())
        K_all = np.concatenate([K_all, C.host(kn)], axis=2)
        step = RetrievalStep(mem, w.n_q_heads, 1, w.k, w.sinks, w.window, want_lse=True)
        r = AS.refresh()
        built.append(r)
        if r[1] > r[0]:
            at_build[r] = AS.mass.cpu().numpy().astype(np.float64)
        step.run(q, q[:, :, -1, :].contiguous())
        AS.accumulate(q, step.lse)
        torch.cuda.synchronize()
        N = mem.length
        idx = step.idx.cpu().numpy()
        qh = C.host(q)
        for b in range(w.batch):
            for h in range(w.n_q_heads):
                g = h // G
                T = O.attended_mask(N, w.block, w.sinks, w.window, idx[b, h])
                oracle_mass[b, g, :N] += O.window_mass(qh[b, h][None], K_all[b, g, :N], T, step.scale, w.window)
    mass = AS.mass.cpu().numpy()
    assert np.allclose(mass, oracle_mass, rtol=MASS_RTOL, atol=MASS_ATOL), np.abs(mass - oracle_mass).max()
    # representatives: every block built during the loop, from the mass at the time it was built
    assert at_build, "the window moved past at least one block"
    reps = C.host(mem.reps)
    for (r0, r1), mb in at_build.items():
        assert mb[:, :, r0 * w.block:(r0 + 1) * w.block].any(), "the block's tokens received attention"
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                want = O.reps_attnscore(K_all[b, g], mb[b, g], w.block, w.reps_per_block, list(range(r0, r1)))
                assert np.array_equal(reps[b, g, r0:r1], want), (b, g, r0, r1)
