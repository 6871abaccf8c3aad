"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Cases span several tiles and ragged tails at oracle-friendly sizes, the five
workloads at full size (sampled outputs where the oracle would be slow), and
the edge cases of the method: k above the candidate count, no candidates,
caller-made selections with duplicates / -1 / out-of-range entries, several
queries per call, 8 query heads per kv head, head dims served by the generic
kernels, ties and NaN in selection, and run-to-run determinism.
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
SMALL = {
    "tiny": W["tiny_decode"],
    "landmark": W["landmark_decode_32k"].scaled(n_q_heads=4, n_kv_heads=4, n_tokens=3018),
    "infllm": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=8192 + 37, window=512,
                                                  k=8, planted_per_head=2),
    "retrieval": W["retrievalattn_gqa_decode_1m_b8"].scaled(batch=2, n_q_heads=8, n_kv_heads=2, n_tokens=16384,
                                                             k=32),
    "memlong": W["memlong_chunk_prefill_80k"].scaled(n_q_heads=4, n_kv_heads=4, n_tokens=8 * 512 + 512),
    "gqa8": W["infllm_gqa_decode_128k"].scaled(n_q_heads=16, n_kv_heads=2, n_tokens=4096 + 100, window=256,
                                                sinks=64, k=6, planted_per_head=1),
    "multi_q": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=6000, window=300, k=5,
                                                   n_q=3, planted_per_head=0),
    "bf16_d64": W["retrievalattn_gqa_decode_1m_b8"].scaled(batch=1, n_q_heads=4, n_kv_heads=4, head_dim=64,
                                                            rep_dim=64, n_tokens=5000, k=12, window=100, sinks=3),
    "bf16_d96_generic": W["retrievalattn_gqa_decode_1m_b8"].scaled(batch=1, n_q_heads=6, n_kv_heads=2,
                                                                    head_dim=96, rep_dim=96, n_tokens=3333, k=7,
                                                                    window=200, sinks=5, block=32),
    "f32_d48_generic": W["tiny_decode"].scaled(n_q_heads=2, n_kv_heads=1, head_dim=48, rep_dim=48, n_tokens=2500,
                                                block=40, k=6),
    "f32_topnorm": W["tiny_decode"].scaled(n_q_heads=4, n_kv_heads=2, rep_mode="topnorm", reps_per_block=3,
                                            n_tokens=3000, block=50, k=5, window=64, sinks=10),
    # 800 selection entries per kv slice (4 heads x k = 200): the wide slot layout (up to 1280 entries)
    "retrieval_wide": W["retrievalattn_gqa_decode_1m_b8"].scaled(batch=1, n_q_heads=8, n_kv_heads=2,
                                                                  n_tokens=16384 + 5, block=16, k=200),
    # two query heads per kv head: two selecting waves, six taking the sink/window tiles
    "gqa2": W["infllm_gqa_decode_128k"].scaled(n_q_heads=4, n_kv_heads=2, n_tokens=5000 + 3, window=300, k=7,
                                               planted_per_head=2),
    # chunks of queries on the matrix-core prefill kernel (n_q >= 64, bf16, head_dim <= 128)
    "prefill_gqa": W["infllm_gqa_decode_128k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=6000 + 11, block=64,
                                                       window=200, sinks=16, k=5, n_q=100, planted_per_head=0),
    "prefill_d64_short_window": W["retrievalattn_gqa_decode_1m_b8"].scaled(
        batch=2, n_q_heads=4, n_kv_heads=4, head_dim=64, rep_dim=64, n_tokens=4000, block=32, k=10, window=40,
        n_q=150),
    # 250 selected 16-token blocks per head: 252 segments, the most one prefill workgroup holds
    "prefill_many_segments": W["infllm_gqa_decode_128k"].scaled(n_q_heads=4, n_kv_heads=2, n_tokens=300 * 16 + 7,
                                                                 block=16, window=64, sinks=8, k=250, n_q=64,
                                                                 planted_per_head=0),
    # the prefill kernel requests its first four 64-token stages before the
    # segments are built when the first segment covers them: sinks first
    # (300 sink tokens), a selected 300-token block first (no sinks), the
    # window first (every token in the window, so no candidate blocks)
    "prefill_first_segment_sinks": W["infllm_gqa_decode_128k"].scaled(
        n_q_heads=4, n_kv_heads=2, n_tokens=5000 + 9, block=64, window=128, sinks=300, k=6, n_q=80,
        planted_per_head=0),
    "prefill_first_segment_block": W["memlong_chunk_prefill_80k"].scaled(
        n_q_heads=2, n_kv_heads=2, head_dim=128, row_stride=128, n_tokens=20 * 300 + 77, block=300, window=400,
        k=4, n_q=96),
    "prefill_first_segment_window": W["infllm_gqa_decode_128k"].scaled(
        n_q_heads=4, n_kv_heads=2, n_tokens=3000, block=64, window=3000, sinks=0, k=4, n_q=70,
        planted_per_head=0),
    # a query chunk with more selected blocks than the prefill kernel's
    # segment table holds (k + 2 > 256): the split path with row groups of
    # 16 query rows takes it
    "prefill_k_past_segment_table": W["infllm_gqa_decode_128k"].scaled(
        n_q_heads=4, n_kv_heads=2, n_tokens=400 * 16 + 7, block=16, window=64, sinks=8, k=300, n_q=64,
        planted_per_head=0),
}


def run_step(mem, w, x, k=None, sinks=None, window=None, scale=None):
    from block_retrieval_sparse_amd.pipeline import RetrievalStep

    step = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k if k is None else k, w.sinks if sinks is None else sinks,
                         w.window if window is None else window, scale=scale)
    qrep = x["rq"] if w.rep_mode == "embed" else x["q"][:, :, -1, :].contiguous()
    step.run(x["q"], qrep)
    return step


@pytest.mark.parametrize("name", list(SMALL))
def test_append_and_reps(name):
    w = SMALL[name]
    mem, x = C.load(w, pieces=3)
    torch.cuda.synchronize()
    N, d = w.n_tokens, w.head_dim
    assert mem.length == N
    assert torch.equal(mem.k[:, :, :N, :d], x["k"]) and torch.equal(mem.v[:, :, :N, :d], x["v"])
    if w.stride > d:
        assert not mem.k[:, :, :N, d:].any() and not mem.v[:, :, :N, d:].any()
    C.check_reps(w, mem, C.oracle_reps(w, x))


@pytest.mark.parametrize("name", list(SMALL))
def test_step(name):
    w = SMALL[name]
    mem, x = C.load(w)
    step = run_step(mem, w, x)
    res = C.check_step(w, mem, x, step)
    print(f"{name}: max |err| {res['max_abs_err']:.3g}")
    if w.planted_per_head:
        idx = step.idx.cpu().numpy()
        for (b, h), blocks in x["planted"].items():
            assert set(blocks) <= set(idx[b, h].tolist()), (b, h)


@pytest.mark.parametrize("name", ["prefill_gqa", "memlong", "infllm", "bf16_d64"])
@pytest.mark.parametrize("scale", [-0.3, 1.5])
def test_step_softmax_scale(name, scale):
    """A negative softmax scale, and a large one (attention close to one-hot,
    where the precision of the weights matters most)."""
    w = SMALL[name]
    mem, x = C.load(w)
    step = run_step(mem, w, x, scale=scale)
    res = C.check_step(w, mem, x, step)
    print(f"{name} scale {scale}: max |err| {res['max_abs_err']:.3g}")


@pytest.mark.parametrize("kind", ["equal", "few", "nan", "quantized"])
def test_step_selection_ties_and_nan(kind):
    """The decode step selects inside its attention kernel; scores with many
    exact ties (every block equal, three distinct representatives, rounded
    representatives) and NaN scores must give the oracle's selection (ties to
    the lowest block index, NaN last) and the same bits as the standalone
    selection followed by the attention call."""
    from block_retrieval_sparse_amd.pipeline import RetrievalStep
    from synth import inputs as I

    w = W["landmark_decode_32k"].scaled(n_q_heads=8, n_kv_heads=2, n_tokens=40000 + 17, k=32)
    x = I.make_all(w, "cuda")
    reps = x["given_reps"]
    g = torch.Generator(device="cpu").manual_seed(7)
    if kind == "equal":
        reps[:] = reps[:, :, :1]
    elif kind == "few":
        pick = torch.randint(0, 3, (reps.shape[2],), generator=g).to(reps.device)
        reps[:] = reps[:, :, :3][:, :, pick]
    elif kind == "nan":
        bad = torch.randint(0, reps.shape[2], (40,), generator=g).to(reps.device)
        reps[:, :, bad] = float("nan")
    else:
        reps[:] = (reps.float() * 2).round().to(reps.dtype) / 2
    mem, x = C.load(w, x=x)
    step = run_step(mem, w, x)
    C.check_step(w, mem, x, step, check_scores=kind != "nan")  # NaN payloads are not compared
    three = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k, w.sinks, w.window)
    three.run_separate(x["q"], x["q"][:, :, -1, :].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(step.idx, three.idx)
    assert torch.equal(step.vals.nan_to_num(0), three.vals.nan_to_num(0))
    assert torch.equal(step.out, three.out)


def test_determinism():
    w = SMALL["retrieval"]
    mem, x = C.load(w)
    a = run_step(mem, w, x)
    outs = (a.scores.clone(), a.idx.clone(), a.out.clone())
    b = run_step(mem, w, x)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].nan_to_num(0), b.scores.nan_to_num(0))
    assert torch.equal(outs[1], b.idx)
    assert torch.equal(outs[2], b.out)


def test_k_above_candidates_and_no_candidates():
    w = SMALL["landmark"]
    mem, x = C.load(w)
    lo, hi = mem.eligible_range(w.sinks, w.window)
    wk = w.scaled(k=hi - lo + 9)
    step = run_step(mem, wk, x)
    C.check_step(wk, mem, x, step)
    assert (step.idx[:, :, hi - lo:] == -1).all()
    # a window covering all tokens leaves no candidate: plain causal attention
    wn = w.scaled(window=w.n_tokens)
    step = run_step(mem, wn, x)
    assert step.lo == step.hi
    C.check_step(wn, mem, x, step)


@pytest.mark.parametrize("case", ["many_blocks", "fewer_than_k", "all_equal"])
def test_cosine_prefill_selection_cases(case):
    """MemLong chunked prefill: scores bit-exact, selection and attention
    against the oracle, with 700 candidate blocks; with fewer candidates than
    k (-1 / -inf tail); with every embedding equal (all scores tied, more than
    the fast selection ranks: the lowest block indices win)."""
    from synth import inputs as I

    base = W["memlong_chunk_prefill_80k"]
    small = dict(n_q_heads=2, n_kv_heads=2, head_dim=64, row_stride=64, block=64, window=64, n_q=64)
    if case == "many_blocks":
        w = base.scaled(n_tokens=700 * 64 + 64, k=20, **small)
    elif case == "fewer_than_k":
        w = base.scaled(n_q_heads=2, n_kv_heads=2, n_tokens=4 * 512 + 512, k=5, n_q=64)
    else:
        w = base.scaled(n_tokens=400 * 64 + 64, k=16, **small)
    x = I.make_all(w, "cuda")
    if case == "all_equal":
        x["embeds"][:] = x["embeds"][:, :, :1]
        x["rq"] = x["embeds"][:, :, -1, 0, :].contiguous()
    mem, x = C.load(w, x=x)
    step = run_step(mem, w, x)
    C.check_step(w, mem, x, step, query_rows=[0, 31, 63])
    lo, hi = step.lo, step.hi
    idx, vals, sc = step.idx.cpu().numpy(), step.vals.cpu().numpy(), step.scores.cpu().numpy()
    m = min(w.k, hi - lo)
    for b in range(w.batch):
        assert np.array_equal(vals[b, 0, :m].view(np.uint32), sc[b, 0, idx[b, 0, :m]].view(np.uint32))
        assert (idx[b, 0, m:] == -1).all() and np.isneginf(vals[b, 0, m:]).all()
        if case == "all_equal":
            assert np.array_equal(idx[b, 0], np.arange(lo, lo + w.k))
    if case == "fewer_than_k":
        assert hi - lo < w.k


@pytest.mark.parametrize("name", ["infllm", "prefill_gqa"])
def test_caller_selection_with_duplicates_and_skips(name):
    """Selections from the caller: duplicates count once, -1 and out-of-range
    entries are skipped, blocks overlapping sinks/window are deduplicated
    (decode, and the chunked prefill, whose workgroups build each head's
    segments from the selection themselves; there the heads of a group get
    different lists, with blocks across and inside the window)."""
    w = SMALL[name]
    mem, x = C.load(w)
    nb = w.n_blocks
    base = [5, 5, -1, nb, nb + 100, 0, nb - 1, 3]
    if w.n_q > 1:
        wb = (w.n_tokens - w.window) // w.block  # the block the window starts in
        base += [wb, wb + 1, wb - 1, wb - 1, nb - 2, 17, 2 ** 31 - 1, -7]
    rows = [base[h % len(base):] + base[:h % len(base)] for h in range(w.n_q_heads)]
    idx = torch.tensor([rows] * w.batch, dtype=torch.int32, device="cuda")
    out = mem.retrieval_attention(x["q"], idx, w.sinks, w.window)
    torch.cuda.synchronize()
    q, K, V = C.host(x["q"]), C.host(x["k"]), C.host(x["v"])
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            g = h // w.group
            T = O.attended_mask(w.n_tokens, w.block, w.sinks, w.window, idx[b, h].tolist())
            ref = O.attention(q[b, h], K[b, g], V[b, g], T, C.scale_of(w))
            assert np.max(np.abs(out[b, h].cpu().numpy() - ref)) <= C.TOL[w.dtype], (b, h)


def test_wide_caller_selection_with_repeats():
    """1000 caller-made entries per kv slice (4 heads x 250, the wide slot
    layout): random blocks with repeats within and across heads, -1 and
    out-of-range entries; each head's output against the oracle on its own
    attended set."""
    w = SMALL["retrieval_wide"]
    mem, x = C.load(w)
    nb = w.n_blocks
    rng = np.random.default_rng(2024)
    idx = torch.from_numpy(rng.integers(-3, nb + 3, size=(w.batch, w.n_q_heads, 250)).astype(np.int32)).cuda()
    out = mem.retrieval_attention(x["q"], idx, w.sinks, w.window)
    torch.cuda.synchronize()
    q, K, V = C.host(x["q"]), C.host(x["k"]), C.host(x["v"])
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            g = h // w.group
            T = O.attended_mask(w.n_tokens, w.block, w.sinks, w.window, idx[b, h].tolist())
            ref = O.attention(q[b, h], K[b, g], V[b, g], T, C.scale_of(w))
            assert np.max(np.abs(out[b, h].cpu().numpy() - ref)) <= C.TOL[w.dtype], (b, h)


def test_empty_set_gives_zeros_and_static_empty_is_an_error():
    import block_retrieval_sparse_amd as brs

    w = SMALL["retrieval"]
    mem, x = C.load(w)
    idx = torch.full((w.batch, w.n_q_heads, 4), -1, dtype=torch.int32, device="cuda")
    out = mem.retrieval_attention(x["q"], idx, 0, 0)
    torch.cuda.synchronize()
    assert not out.any()
    with pytest.raises(brs.BrsError) as e:
        mem.retrieval_attention(x["q"], None, 0, 0)
    assert e.value.code == -5


@pytest.mark.parametrize("name", ["infllm", "prefill_gqa"])
def test_broadcast_selection_dot_mode(name):
    """One selection per sequence (idx_heads = 1) in dot mode."""
    w = SMALL[name]
    mem, x = C.load(w)
    idx = torch.tensor([[[7, 2, 40, 11]]] * w.batch, dtype=torch.int32, device="cuda")
    out = mem.retrieval_attention(x["q"], idx, w.sinks, w.window)
    torch.cuda.synchronize()
    q, K, V = C.host(x["q"]), C.host(x["k"]), C.host(x["v"])
    T = O.attended_mask(w.n_tokens, w.block, w.sinks, w.window, [7, 2, 40, 11])
    for h in range(w.n_q_heads):
        ref = O.attention(q[0, h], K[0, h // w.group], V[0, h // w.group], T, C.scale_of(w))
        assert np.max(np.abs(out[0, h].cpu().numpy() - ref)) <= C.TOL[w.dtype]


@pytest.mark.parametrize("n,k,kind", [(1, 1, "normal"), (60, 4, "ties"), (991, 32, "ties"), (991, 32, "nan"),
                                      (5000, 2048, "normal"), (16384, 320, "ties"), (16384, 320, "zeros"),
                                      (20000, 100, "ties"), (700, 700, "normal"), (50, 64, "normal"),
                                      (1500, 100, "ties"), (2048, 512, "normal"), (2048, 513, "ties"),
                                      (130, 33, "nan"),
                                      # one 1024-thread workgroup per row (radix select), keys in registers
                                      (3000, 100, "normal"), (3000, 64, "nan"), (10000, 512, "ties"),
                                      (16384, 1, "normal"), (4096, 200, "zeros"), (12000, 333, "ties"),
                                      (8000, 300, "mostly_nan"),
                                      # the keys at or above the digits found so far ranked directly
                                      # once at most 2k: after the first pass (normal), after later
                                      # ones (scores within a narrow band), at the 2048-key gather
                                      # limit (2k = 2048), never (k = 2048), and with k <= 64
                                      (16384, 320, "normal"), (16384, 320, "near"), (16384, 1024, "normal"),
                                      (16384, 2048, "ties"), (5000, 40, "normal"), (16384, 700, "nan")])
def test_select_topk(n, k, kind):
    import block_retrieval_sparse_amd as brs

    rng = np.random.default_rng(n + k)
    rows, stride, lo = 3, n + 11, 5
    s = rng.standard_normal((rows, stride)).astype(np.float32)
    if kind == "ties":
        s = np.round(s * 4) / 4
    if kind == "near":  # one exponent, few distinct leading mantissa bits
        s = (3.0 + 0.05 * s).astype(np.float32)
    if kind == "nan":
        s[:, rng.integers(0, stride, 40)] = np.nan
    if kind == "mostly_nan":  # fewer numbers than k: the k-th key is NaN's
        s[rng.random((rows, stride)) < 0.97] = np.nan
    if kind == "zeros":
        s = np.where(rng.random((rows, stride)) < 0.5, np.float32(0.0), np.float32(-0.0))
        s[rng.random((rows, stride)) < 0.01] = 1.0
    hi = lo + n
    st = torch.from_numpy(s).cuda()[None].reshape(1, rows, stride).contiguous()
    idx, vals = brs.select_topk(st, lo, hi, k)
    torch.cuda.synchronize()
    for r in range(rows):
        oi, ov = O.select_topk(s[r], lo, hi, k)
        assert np.array_equal(idx[0, r].cpu().numpy(), oi), (r, idx[0, r][:10], oi[:10])
        gv = vals[0, r].cpu().numpy()
        assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32)) or np.array_equal(gv, ov, equal_nan=True)


# ---------------------------------------------------------------------------
# the five workloads at full size


@pytest.mark.parametrize("name", ["tiny_decode", "landmark_decode_32k", "infllm_gqa_decode_128k"])
def test_full_size_decode(name):
    w = W[name]
    mem, x = C.load(w)
    step = run_step(mem, w, x)
    res = C.check_step(w, mem, x, step)
    print(f"{name}: max |err| {res['max_abs_err']:.3g}")
    for (b, h), blocks in x["planted"].items():
        assert set(blocks) <= set(step.idx[b, h].cpu().tolist())


def test_full_size_retrievalattn_sampled():
    w = W["retrievalattn_gqa_decode_1m_b8"]
    mem, x = C.load(w)
    step = run_step(mem, w, x)
    pairs = [(0, 0), (3, 13), (7, 31), (5, 22)]
    res = C.check_step(w, mem, x, step, pairs=pairs)
    print(f"retrievalattn: max |err| {res['max_abs_err']:.3g}")


def test_full_size_memlong_prefill_sampled():
    w = W["memlong_chunk_prefill_80k"]
    mem, x = C.load(w)
    step = run_step(mem, w, x)
    res = C.check_step(w, mem, x, step, pairs=[(0, 0), (0, 17), (0, 31)],
                       query_rows=[0, 1, 63, 64, 255, 448, 510, 511])
    print(f"memlong: max |err| {res['max_abs_err']:.3g}")


@pytest.mark.parametrize("name", ["infllm", "gqa8", "gqa2", "landmark", "retrieval", "retrieval_wide", "memlong",
                                  "multi_q", "prefill_gqa"])
def test_step_call_matches_separate_calls(name):
    """brs_retrieval_step (one call; for decode the attention kernel makes the
    selection itself) gives the same scores, selection and attention bits as
    the three separate calls."""
    from block_retrieval_sparse_amd.pipeline import RetrievalStep

    w = SMALL[name]
    mem, x = C.load(w)
    qrep = x["rq"] if w.rep_mode == "embed" else x["q"][:, :, -1, :].contiguous()
    one = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k, w.sinks, w.window)
    three = RetrievalStep(mem, w.n_q_heads, w.n_q, w.k, w.sinks, w.window)
    one.run(x["q"], qrep)
    three.run_separate(x["q"], qrep)
    torch.cuda.synchronize()
    lo, hi = one.lo, one.hi
    assert torch.equal(one.scores[:, :, lo:hi], three.scores[:, :, lo:hi])
    assert torch.equal(one.idx, three.idx)
    assert torch.equal(one.vals, three.vals)
    assert torch.equal(one.out, three.out)
